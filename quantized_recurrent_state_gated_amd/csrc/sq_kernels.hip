// sq_kernels.hip -- gfx950 kernels of the fused quantized gated delta-rule
// decode step.
//
// Sources (cited by title and section):
//   [P1] "K1 論文詳解" (k1-news, 2026-10-09), STEPQuant article, 方法.
//   [P5] "线性注意力状态量化难题:Qwen状态池70并发就超模型权重" (aitest123),
//        直接量化为什么会翻车, 时间维度, 空间维度, 工程落地.
//
// The step is one rank-1 update per (request, head) tile, so it is bound by
// HBM bandwidth, not by arithmetic: the pages fuse quantization with the state
// update precisely to cut memory traffic ([P1] 方法, last paragraph; [P5]
// 工程落地).  Here every tile is streamed from HBM once and written back once;
// there is no MFMA (nothing here is a dense contraction).
//
// Arithmetic is done in the code domain.  With Shat_ij = q_ij r_i c_j and the
// update S' = alpha Shat + beta k (v - alpha u)^T, u = Shat^T k:
//     u_j  = c_j * sum_i (k_i r_i) q_ij                 (column reduction)
//     y_j  = c_j * sum_i (q_i r_i) q_ij                 (readout of Shat)
//     S'_ij / (r_i c_j) = alpha q_ij + a_i b_j,  a_i = beta k_i / r_i,
//                                                 b_j = (v_j - alpha u_j) / c_j
//     o_j  = alpha y_j + beta (q.k) (v_j - alpha u_j)   ( = sum_i q_i S'_ij )
// so the tile is touched by two fused multiply-adds per element per pass and
// o needs no second reduction.  Codes are carried in their stored excess form
// n = q + 2^(b-1); the bias is folded into per-tile constants.
//
// The per-key-channel gate (the KDA reading, [P5] 直接量化为什么会翻车:
// S' = (I - beta k k^T) diag(alpha) Shat + beta k v^T, alpha in R^{d_k}) is
// the same arithmetic with alpha_i moved into the row factors: u and y use
// weights alpha_i k_i r_i and alpha_i q_i r_i, the column terms take alpha = 1,
// and the requantization uses alpha_i per row.  Template flag CHG.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <mutex>
#include <type_traits>
#include <utility>
#include <stdint.h>

#include "sq_launch.h"

namespace sqk {

// ---------------------------------------------------------------- loads

template <typename T>
__device__ __forceinline__ float ld1(const T *p, long i);
template <>
__device__ __forceinline__ float ld1<float>(const float *p, long i) { return p[i]; }
template <>
__device__ __forceinline__ float ld1<uint16_t>(const uint16_t *p, long i)
{
    return __uint_as_float((uint32_t)p[i] << 16);  // bf16 -> fp32 is exact
}

template <typename T>
__device__ __forceinline__ void ld4(const T *p, long i, float (&x)[4]);
template <>
__device__ __forceinline__ void ld4<float>(const float *p, long i, float (&x)[4])
{
    float4 f = *reinterpret_cast<const float4 *>(p + i);
    x[0] = f.x; x[1] = f.y; x[2] = f.z; x[3] = f.w;
}
template <>
__device__ __forceinline__ void ld4<uint16_t>(const uint16_t *p, long i, float (&x)[4])
{
    uint2 u = *reinterpret_cast<const uint2 *>(p + i);
    x[0] = __uint_as_float(u.x << 16);
    x[1] = __uint_as_float(u.x & 0xffff0000u);
    x[2] = __uint_as_float(u.y << 16);
    x[3] = __uint_as_float(u.y & 0xffff0000u);
}

// ---------------------------------------------------------------- block codec
//
// A 4x4 block is 16 consecutive fields, field e = 4*col + row, packed LSB
// first; it is BITS/2 dwords long.  decode() yields each field as a float:
// the excess-form code n for 4/6/8 bits, the value itself for 16/32 bits.
// encode() takes the updated value in the same form; codes are clamped to
// [1, 2^b - 1] (the symmetric range) and rounded half to even.

// Format tags are the head_bits values: 4, 6, 8 (codes), 16 (FP16 pivot),
// 32 (FP32 state) and kBF16 (bfloat16 state).  fw<F>() is the field width.
constexpr int kBF16 = 144;

template <int F>
constexpr int fw()
{
    return F == kBF16 ? 16 : F;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int BITS>
__device__ __forceinline__ void decode(const uint32_t (&d)[fw<BITS>() / 2], float (&f)[16])
{
    if constexpr (BITS == 8) {
#pragma unroll
        for (int e = 0; e < 16; e++) f[e] = (float)((d[e >> 2] >> (8 * (e & 3))) & 0xffu);
    } else if constexpr (BITS == 4) {
        // split each dword's nibbles into two dwords of bytes, then convert
        // bytes directly (v_cvt_f32_ubyte0..3); the empty asm keeps the
        // compiler from folding the masks back into per-field bit extracts
#pragma unroll
        for (int w = 0; w < 2; w++) {
            uint32_t lo = d[w] & 0x0f0f0f0fu, hi = (d[w] >> 4) & 0x0f0f0f0fu;
            asm volatile("" : "+v"(lo), "+v"(hi));
#pragma unroll
            for (int p = 0; p < 4; p++) {
                f[8 * w + 2 * p] = (float)((lo >> (8 * p)) & 0xffu);
                f[8 * w + 2 * p + 1] = (float)((hi >> (8 * p)) & 0xffu);
            }
        }
    } else if constexpr (BITS == 6) {
#pragma unroll
        for (int e = 0; e < 16; e++) {
            const int bit = 6 * e, w = bit >> 5, s = bit & 31;
            uint32_t x;
            if (s + 6 <= 32)
                x = d[w] >> s;
            else
                x = (d[w] >> s) | (d[w + 1] << (32 - s));
            f[e] = (float)(x & 0x3fu);
        }
    } else if constexpr (BITS == 16) {
#pragma unroll
        for (int e = 0; e < 16; e++)
            f[e] = __half2float(__ushort_as_half((unsigned short)(d[e >> 1] >> (16 * (e & 1)))));
    } else if constexpr (BITS == kBF16) {
        // a bfloat16 is the upper half of a binary32
#pragma unroll
        for (int e = 0; e < 16; e++)
            f[e] = __uint_as_float((e & 1) ? (d[e >> 1] & 0xffff0000u) : (d[e >> 1] << 16));
    } else {
#pragma unroll
        for (int e = 0; e < 16; e++) f[e] = __uint_as_float(d[e]);
    }
}

// v_cvt_pk_u8_f32: convert x to an unsigned byte (round half to even,
// saturating to [0, 255]) and insert it as byte `sel` of `acc`.
__device__ __forceinline__ uint32_t pk_u8(float x, uint32_t sel, uint32_t acc)
{
    return __builtin_amdgcn_cvt_pk_u8_f32(x, sel, acc);
}

template <int BITS>
__device__ __forceinline__ float clamp_code(float z)
{
    // symmetric range [1, 2^b - 1] in excess form; the upper bound of the
    // 8-bit range is the conversion's own saturation.  Callers map a NaN to
    // code 0 (OFF) before this.
    if constexpr (BITS == 8) return fmaxf(z, 1.0f);
    else return __builtin_amdgcn_fmed3f(z, 1.0f, (float)((1 << BITS) - 1));
}

template <int BITS>
__device__ __forceinline__ void encode(const float (&z)[16], uint32_t (&d)[fw<BITS>() / 2])
{
    if constexpr (BITS == 8) {
#pragma unroll
        for (int w = 0; w < 4; w++) {
            uint32_t x = pk_u8(clamp_code<8>(z[4 * w]), 0, 0u);
            x = pk_u8(clamp_code<8>(z[4 * w + 1]), 1, x);
            x = pk_u8(clamp_code<8>(z[4 * w + 2]), 2, x);
            d[w] = pk_u8(clamp_code<8>(z[4 * w + 3]), 3, x);
        }
    } else if constexpr (BITS == 4) {
        // even fields into one dword of bytes, odd fields into another, then
        // interleave the nibbles with one shift-or
#pragma unroll
        for (int w = 0; w < 2; w++) {
            uint32_t ev = 0u, od = 0u;
#pragma unroll
            for (int p = 0; p < 4; p++) {
                ev = pk_u8(clamp_code<4>(z[8 * w + 2 * p]), p, ev);
                od = pk_u8(clamp_code<4>(z[8 * w + 2 * p + 1]), p, od);
            }
            d[w] = ev | (od << 4);
        }
    } else if constexpr (BITS == 6) {
        // four codes of a column -> four bytes (each < 64) -> one 24-bit group
        // f0 | f1 << 6 | f2 << 12 | f3 << 18, as two byte dot products
        // (f0 + 64 f1 and f2 + 64 f3) joined by a shift-or; the four 3-byte
        // groups are then spliced into three dwords with byte permutes
        uint32_t g[4];
#pragma unroll
        for (int c = 0; c < 4; c++) {
            uint32_t x = pk_u8(clamp_code<6>(z[4 * c]), 0, 0u);
            x = pk_u8(clamp_code<6>(z[4 * c + 1]), 1, x);
            x = pk_u8(clamp_code<6>(z[4 * c + 2]), 2, x);
            x = pk_u8(clamp_code<6>(z[4 * c + 3]), 3, x);
            const uint32_t lo12 = __builtin_amdgcn_udot4(x, 0x00004001u, 0u, false);
            const uint32_t hi12 = __builtin_amdgcn_udot4(x, 0x40010000u, 0u, false);
            g[c] = lo12 | (hi12 << 12);
        }
        d[0] = __builtin_amdgcn_perm(g[1], g[0], 0x04020100u);  // g0 bytes 0-2, g1 byte 0
        d[1] = __builtin_amdgcn_perm(g[2], g[1], 0x05040201u);  // g1 bytes 1-2, g2 bytes 0-1
        d[2] = __builtin_amdgcn_perm(g[3], g[2], 0x06050402u);  // g2 byte 2, g3 bytes 0-2
    } else if constexpr (BITS == 16) {
#pragma unroll
        for (int w = 0; w < 8; w++) {
            const uint32_t lo = __half_as_ushort(__float2half_rn(z[2 * w]));
            const uint32_t hi = __half_as_ushort(__float2half_rn(z[2 * w + 1]));
            d[w] = lo | (hi << 16);
        }
    } else if constexpr (BITS == kBF16) {
        // round half to even, two values per conversion (v_cvt_pk_bf16_f32)
#pragma unroll
        for (int w = 0; w < 8; w++) {
            const f32x2 x = {z[2 * w], z[2 * w + 1]};
            d[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
        }
    } else {
#pragma unroll
        for (int e = 0; e < 16; e++) d[e] = __float_as_uint(z[e]);
    }
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) uint8_t gbyte;  // global memory

// Tile blocks are streamed: read once, written once, never reused by this
// launch, so they may bypass cache retention (nontemporal hint).
template <int BITS, bool NT, typename B>
__device__ __forceinline__ void load_block(const B *p, uint32_t (&d)[fw<BITS>() / 2])
{
    using U2 = typename std::conditional<std::is_same<B, gbyte>::value,
                                         const __attribute__((address_space(1))) u32x2, const u32x2>::type;
    using U1 = typename std::conditional<std::is_same<B, gbyte>::value,
                                         const __attribute__((address_space(1))) uint32_t, const uint32_t>::type;
    using U4 = typename std::conditional<std::is_same<B, gbyte>::value,
                                         const __attribute__((address_space(1))) u32x4, const u32x4>::type;
    if constexpr (BITS == 4) {
        U2 *q = reinterpret_cast<U2 *>(p);
        const u32x2 x = NT ? __builtin_nontemporal_load(q) : *q;
        d[0] = x.x; d[1] = x.y;
    } else if constexpr (BITS == 6) {
        U1 *q = reinterpret_cast<U1 *>(p);
#pragma unroll
        for (int w = 0; w < 3; w++) d[w] = NT ? __builtin_nontemporal_load(q + w) : q[w];
    } else {
#pragma unroll
        for (int w = 0; w < fw<BITS>() / 2; w += 4) {
            U4 *q = reinterpret_cast<U4 *>(p + 4 * w);
            const u32x4 x = NT ? __builtin_nontemporal_load(q) : *q;
            d[w] = x.x; d[w + 1] = x.y; d[w + 2] = x.z; d[w + 3] = x.w;
        }
    }
}

template <int BITS, bool NT, typename B>
__device__ __forceinline__ void store_block(B *p, const uint32_t (&d)[fw<BITS>() / 2])
{
    using U2 = typename std::conditional<std::is_same<B, gbyte>::value,
                                         __attribute__((address_space(1))) u32x2, u32x2>::type;
    using U1 = typename std::conditional<std::is_same<B, gbyte>::value,
                                         __attribute__((address_space(1))) uint32_t, uint32_t>::type;
    using U4 = typename std::conditional<std::is_same<B, gbyte>::value,
                                         __attribute__((address_space(1))) u32x4, u32x4>::type;
    if constexpr (BITS == 4) {
        U2 *q = reinterpret_cast<U2 *>(p);
        const u32x2 x = {d[0], d[1]};
        if (NT) __builtin_nontemporal_store(x, q); else *q = x;
    } else if constexpr (BITS == 6) {
        U1 *q = reinterpret_cast<U1 *>(p);
#pragma unroll
        for (int w = 0; w < 3; w++) {
            if (NT) __builtin_nontemporal_store(d[w], q + w); else q[w] = d[w];
        }
    } else {
#pragma unroll
        for (int w = 0; w < fw<BITS>() / 2; w += 4) {
            U4 *q = reinterpret_cast<U4 *>(p + 4 * w);
            const u32x4 x = {d[w], d[w + 1], d[w + 2], d[w + 3]};
            if (NT) __builtin_nontemporal_store(x, q); else *q = x;
        }
    }
}

// Sum over the 64 lanes of a wave with DPP row operations; the total is
// returned in every lane (read back from lane 63).
__device__ __forceinline__ float dpp_add(float x, float y) { return x + y; }

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, false));
}

__device__ __forceinline__ float wave_sum(float x)
{
    x += dpp<0xb1>(x);        // quad_perm [1,0,3,2]
    x += dpp<0x4e>(x);        // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);       // row_half_mirror: sums of 8
    x += dpp<0x140>(x);       // row_mirror: sums of 16
    x += dpp<0x142, 0xa>(x);  // row_bcast15 into rows 1, 3: sums of 32 there
    x += dpp<0x143, 0xc>(x);  // row_bcast31 into rows 2, 3: lane 63 holds the total
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// ---------------------------------------------------------------- XCD-aware tile order
//
// The dispatcher deals workgroups to the 8 XCDs of an MI355X round-robin
// (workgroup g runs on XCD g % 8).  With workgroup g on tile g, the XCDs
// drift apart over a long launch and the eight of them end up streaming from
// scattered parts of one address window; bandwidth then falls with the batch
// (5.84 TB/s at 70 requests x 2304 heads, 5.3 TB/s at 128 and 256).
// Instead XCD x takes a contiguous group of heads, [x H / 8, (x+1) H / 8),
// of every request, request after request: the group's tiles are contiguous
// in each slot's slab, so each XCD streams compact runs, and it reads the
// row and column factors of its own heads only (they stay in its L2).
// Measured: +8-10 % at 128-256 requests, neutral at 70.  With fewer than
// kXcdGroupMin heads a group would leave XCDs idle, so small pools take
// contiguous eighths of the tile range instead.  Surplus workgroups of the
// rounded-up grid exit at once.

constexpr uint32_t kXcds = 8;
constexpr uint32_t kXcdGroupMin = 64;

// floor(i / d) for d >= 1 from m = ceil(2^32 / d) (host-computed, 0 for
// d = 1): umulhi(i, m) is floor(i / d) or one more.
__device__ __forceinline__ uint32_t div_magic(uint32_t i, uint32_t d, uint32_t m)
{
    if (d == 1) return i;
    uint32_t q = __umulhi(i, m);
    if (q * d > i) q--;
    return q;
}

// Tile (n, h) of workgroup blockIdx.x for n_req requests x H heads; false if
// the workgroup has no tile.  xm[x] is the reciprocal of XCD x's head count
// (H >= kXcdGroupMin) or, in xm[0], of H itself (smaller pools).
__device__ __forceinline__ bool xcd_tile(uint32_t n_req, uint32_t H, const uint32_t (&xm)[8],
                                         uint32_t &n, uint32_t &h)
{
    const uint32_t x = blockIdx.x % kXcds, i = blockIdx.x / kXcds;
    if (H >= kXcdGroupMin) {
        const uint32_t h0 = (uint32_t)((uint64_t)x * H / kXcds);
        const uint32_t hx = (uint32_t)((uint64_t)(x + 1) * H / kXcds) - h0;
        n = div_magic(i, hx, xm[x]);
        h = h0 + (i - n * hx);
        return n < n_req;
    }
    const uint32_t total = n_req * H, per = (total + kXcds - 1) / kXcds, b = x * per + i;
    n = div_magic(b, H, xm[0]);
    h = b - n * H;
    return i < per && b < total;
}

__host__ __forceinline__ uint32_t xcd_grid(uint32_t n_req, uint32_t H)
{
    if (H >= kXcdGroupMin) return n_req * ((H + kXcds - 1) / kXcds) * kXcds;
    return (n_req * H + kXcds - 1) / kXcds * kXcds;
}

// Two tiles per workgroup: workgroup g holds the tiles that workgroups
// 2 (g / 8) * 8 + g % 8 and that + 8 would hold alone, i.e. tiles 2i and
// 2i + 1 of XCD g % 8's walk (half = 0, 1).
__device__ __forceinline__ bool xcd_tile_pair(uint32_t n_req, uint32_t H, const uint32_t (&xm)[8],
                                              uint32_t half, uint32_t &n, uint32_t &h)
{
    const uint32_t x = blockIdx.x % kXcds, i = 2 * (blockIdx.x / kXcds) + half;
    if (H >= kXcdGroupMin) {
        const uint32_t h0 = (uint32_t)((uint64_t)x * H / kXcds);
        const uint32_t hx = (uint32_t)((uint64_t)(x + 1) * H / kXcds) - h0;
        n = div_magic(i, hx, xm[x]);
        h = h0 + (i - n * hx);
        return n < n_req;
    }
    const uint32_t total = n_req * H, per = (total + kXcds - 1) / kXcds, b = x * per + i;
    n = div_magic(b, H, xm[0]);
    h = b - n * H;
    return i < per && b < total;
}

__host__ __forceinline__ uint32_t xcd_grid_pair(uint32_t n_req, uint32_t H)
{
    const uint32_t per = H >= kXcdGroupMin ? n_req * ((H + kXcds - 1) / kXcds)
                                           : (n_req * H + kXcds - 1) / kXcds;
    return (per + 1) / 2 * kXcds;
}

static uint32_t magic_of(uint32_t d) { return d <= 1 ? 0u : (uint32_t)(((1ull << 32) + d - 1) / d); }

// the reciprocals xcd_tile needs for H heads
static void xcd_magic(uint32_t H, uint32_t (&xm)[8])
{
    for (uint32_t x = 0; x < kXcds; x++) {
        if (H >= kXcdGroupMin) {
            const uint32_t h0 = (uint32_t)((uint64_t)x * H / kXcds);
            xm[x] = magic_of((uint32_t)((uint64_t)(x + 1) * H / kXcds) - h0);
        } else {
            xm[x] = magic_of(H);
        }
    }
}

// ---------------------------------------------------------------- d = 128 step
//
// Shared memory of one FP32- or BF16-state tile (tile128_wide, 256 threads).

struct SmemWide {
    alignas(16) float w[128];      // per-row factors k_i (times alpha_i with a per-channel gate)
    alignas(16) float g[128];      // q_i (times alpha_i)
    alignas(16) float a[128];      // beta k_i
    alignas(16) float red[8][2][128];  // [row group][u, y][column] partial sums
    alignas(16) float b[128];      // per-column (v_j - alpha u_j) / c_j
    alignas(8) float2 vc[128];     // per-column {v_j, c_j}, staged at the start
    float sum[2][3];               // per-wave partials of q.k, sum w, sum g
};

// Per-key-channel gate: pass 2 needs a per-row gate.  pa[i] = {beta k_i, alpha_i, 0, 0}.
struct SmemWideK : SmemWide {
    alignas(16) float4 pa[128];
};

// tile128_wide: an unquantized FP32 or BF16 state, one 256-thread workgroup
// per tile.  Every load and store instruction of a wave moves one contiguous
// kilobyte: lane l takes the l-th 16-byte chunk of its span.  A 16-byte chunk
// of an FP32 block is one column's four rows, of a BF16 block two columns'
// four rows, so a lane owns CPL = 1 or 2 columns and four rows of every block
// row it visits:
//   FP32: a block row is 2 KB; wave w takes the half ch = w % 2 (columns
//         64 ch + lane) of block rows 16 (w / 2) .. 16 (w / 2) + 15;
//   BF16: a block row is 1 KB; wave w takes block rows 8 w .. 8 w + 7
//         (columns 2 lane and 2 lane + 1).
// A lane's column sums over its 64 rows stay in registers; the two (FP32) or
// four (BF16) row groups are combined through LDS.

// threads per wide tile (measured at 70 x 2304: FP32 states 3.88 ms per step
// with 256, 3.88 with 128, 3.94 with 512; BF16 1.93-1.96 ms for all three)
constexpr int kWideTPB = 256;

template <int FMT, typename T, bool UPDATE, bool CHG, typename SM>
__device__ __forceinline__ void tile128_wide(const StepArgs &a, int n, int h, SM &sm)
{
    static_assert(FMT == 32 || FMT == kBF16, "unquantized states only");
    constexpr int E = FMT == 32 ? 4 : 2;        // bytes per element
    constexpr int CPL = 4 / E;                  // columns per lane
    constexpr int NCH = 128 / (64 * CPL);       // column spans: 2 (FP32) or 1 (BF16)
    constexpr int NRG = kWideTPB / 64 / NCH;    // row groups
    constexpr int NI = 32 / NRG;                // block rows per wave
    static_assert(NRG >= 1 && NRG <= 8 && 32 % NRG == 0, "row groups");
    constexpr int ROW_BYTES = 32 * 16 * E;      // one block row: 2048 or 1024 bytes

    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int ch = wv % NCH, rgp = wv / NCH;
    const long nh = (long)n * a.H + h;
    uint8_t *tile = a.pool + (uint64_t)a.slot_ids[n] * a.slab + (uint64_t)a.head_off[h];
    const T *q = reinterpret_cast<const T *>(a.q);
    const T *k = reinterpret_cast<const T *>(a.k);
    const T *v = reinterpret_cast<const T *>(a.v);

    // with a per-channel gate alpha_i multiplies row i of the weights and the
    // column terms take alpha = 1: u = (diag(alpha) S)^T k, o = y + beta (q.k) (v - u)
    const float alpha = UPDATE && !CHG ? a.alpha[nh] : 1.0f;
    const float beta = UPDATE ? a.beta[nh] : 0.0f;

    // row tr = t % 128 inputs (threads 128..255 repeat rows 0..127) and column
    // tr inputs, loaded before the tile: vector loads complete in issue order,
    // so the row stage does not wait for the tile
    const int tr = t & 127;
    const float qi = ld1(q, nh * 128 + tr);
    const float ki = UPDATE ? ld1(k, nh * 128 + tr) : 0.0f;
    const float gate = CHG ? a.alpha[nh * 128 + tr] : 1.0f;
    const float vj = UPDATE ? ld1(v, nh * 128 + tr) : 0.0f;

    // the lane's chunks: block rows rgp NI + m, m = 0 .. NI - 1
    uint8_t *span = tile + (long)(rgp * NI) * ROW_BYTES + 1024 * ch + 16 * lane;
    uint32_t d[NI][4];
#pragma unroll
    for (int m = 0; m < NI; m++) {
        const u32x4 x = *reinterpret_cast<const u32x4 *>(span + (long)m * ROW_BYTES);
        d[m][0] = x.x; d[m][1] = x.y; d[m][2] = x.z; d[m][3] = x.w;
    }

    {
        sm.w[tr] = ki * gate;
        sm.g[tr] = qi * gate;
        if constexpr (CHG) sm.pa[tr] = make_float4(beta * ki, gate, 0.0f, 0.0f);
        else if (UPDATE) sm.a[tr] = beta * ki;
        sm.vc[tr] = make_float2(vj, 1.0f);
        const float s0 = wave_sum(qi * ki);
        if (t < 128 && (t & 63) == 0) sm.sum[t >> 6][0] = s0;
    }
    __syncthreads();

    // element (row r of the chunk, lane column c) of chunk m
    auto elem = [&](int m, int r, int c) -> float {
        if constexpr (FMT == 32) {
            return __uint_as_float(d[m][r]);
        } else {
            // dword 2c + (r >> 1) holds rows (r & ~1, r | 1) of lane column c
            const uint32_t x = d[m][2 * c + (r >> 1)];
            return __uint_as_float((r & 1) ? (x & 0xffff0000u) : (x << 16));
        }
    };

    // pass 1: this lane's column sums over its 64 rows
    float pu[CPL], py[CPL];
#pragma unroll
    for (int c = 0; c < CPL; c++) pu[c] = py[c] = 0.0f;
#pragma unroll
    for (int m = 0; m < NI; m++) {
        const int i0 = 4 * (rgp * NI + m);
        const float4 w4 = *reinterpret_cast<const float4 *>(&sm.w[i0]);
        const float4 g4 = *reinterpret_cast<const float4 *>(&sm.g[i0]);
        const float wr[4] = {w4.x, w4.y, w4.z, w4.w}, gr[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
        for (int r = 0; r < 4; r++)
#pragma unroll
            for (int c = 0; c < CPL; c++) {
                const float x = elem(m, r, c);
                if (UPDATE) pu[c] = fmaf(wr[r], x, pu[c]);
                py[c] = fmaf(gr[r], x, py[c]);
            }
    }
    const int j0 = CPL * (64 * ch + lane);  // the lane's first column
#pragma unroll
    for (int c = 0; c < CPL; c++) {
        sm.red[rgp][0][j0 + c] = pu[c];
        sm.red[rgp][1][j0 + c] = py[c];
    }
    __syncthreads();

    // column finalisation: thread j < 128 owns column j
    if (t < 128) {
        float U = 0.0f, Y = 0.0f;
#pragma unroll
        for (int r = 0; r < NRG; r++) {
            U += sm.red[r][0][t];
            Y += sm.red[r][1][t];
        }
        const float qk = sm.sum[0][0] + sm.sum[1][0];
        if (!UPDATE) {
            a.o[nh * 128 + t] = Y;
        } else {
            const float e = sm.vc[t].x - alpha * U;
            if (a.o) a.o[nh * 128 + t] = fmaf(alpha, Y, beta * qk * e);
            sm.b[t] = e;
        }
    }
    if (!UPDATE) return;
    __syncthreads();
    float b[CPL];
#pragma unroll
    for (int c = 0; c < CPL; c++) b[c] = sm.b[j0 + c];

    // pass 2: S' = gate S + a_i b_j, rounded to the storage format, stored in
    // place; a non-finite value is recorded in the pool's sticky flag
    bool nf = false;
#pragma unroll
    for (int m = 0; m < NI; m++) {
        const int i0 = 4 * (rgp * NI + m);
        float z[4][CPL];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            float ai, gi;
            if constexpr (CHG) {
                const float4 p = sm.pa[i0 + r];
                ai = p.x;
                gi = p.y;
            } else {
                ai = sm.a[i0 + r];
                gi = alpha;
            }
#pragma unroll
            for (int c = 0; c < CPL; c++) {
                z[r][c] = fmaf(gi, elem(m, r, c), ai * b[c]);
                nf |= !__builtin_isfinite(z[r][c]);
            }
        }
        uint32_t o4[4];
        if constexpr (FMT == 32) {
#pragma unroll
            for (int r = 0; r < 4; r++) o4[r] = __float_as_uint(z[r][0]);
        } else {
            // round half to even, two values per conversion (v_cvt_pk_bf16_f32)
#pragma unroll
            for (int c = 0; c < CPL; c++)
#pragma unroll
                for (int p = 0; p < 2; p++) {
                    const f32x2 x = {z[2 * p][c], z[2 * p + 1][c]};
                    o4[2 * c + p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
                }
        }
        *reinterpret_cast<u32x4 *>(span + (long)m * ROW_BYTES) = u32x4{o4[0], o4[1], o4[2], o4[3]};
    }
    if (__ballot(nf) && lane == 0) atomicOr(a.err, 1);
}

// ---------------------------------------------------------------- packed-half codes
//
// For 4/6/8-bit codes and FP16 pivots a thread keeps its 64 elements as 32
// dwords of packed 16-bit halves.  A code n is placed in the low mantissa
// bits of a half whose exponent field is zero, so the half is exactly the
// binary16 subnormal n * 2^s (s = -24, or -20 where the field sits 4 bits
// up in its half); v_fma_mix_f32 takes it as an exact fp32 operand.  The
// power of two depends on the row of the element only, so it is folded into
// the per-row weights (pass 1) and into the per-row gate (pass 2), and the
// codes need only masks, shifts and byte permutes.  FP16 pivot halves are
// their own values (s = 0).
//
// HalfPos<BITS>: element e = 4*col + row of a block sits in half sel(e) of
// packed dword k(e); row r of the block has the power of two 2^s(r).

template <int BITS>
struct HalfPos;
template <>
struct HalfPos<8> {  // dword 2c + (r & 1) = rows {0,2} or {1,3} of column c
    static constexpr int k(int e) { return 2 * (e >> 2) + (e & 1); }
    static constexpr int sel(int e) { return (e >> 1) & 1; }
    static constexpr int s(int) { return -24; }
};
template <>
struct HalfPos<6> {  // dword 2c + (r & 1): rows {0,2} or {1,3} of column c; rows 0, 1 4 bits up
    static constexpr int k(int e) { return 2 * (e >> 2) + (e & 1); }
    static constexpr int sel(int e) { return (e >> 1) & 1; }
    static constexpr int s(int r) { return r < 2 ? -20 : -24; }
};
template <>
struct HalfPos<4> {  // dword 4(c/2) + r = row r of columns c, c+1; odd rows 4 bits up
    static constexpr int k(int e) { return 4 * (e >> 3) + (e & 3); }
    static constexpr int sel(int e) { return (e >> 2) & 1; }
    static constexpr int s(int r) { return (r & 1) ? -20 : -24; }
};
template <>
struct HalfPos<16> {
    static constexpr int k(int e) { return e >> 1; }
    static constexpr int sel(int e) { return e & 1; }
    static constexpr int s(int) { return 0; }
};

// 2^-s(r): the factor that turns a half of row r back into its code
template <int BITS>
constexpr float unscale(int r)
{
    return HalfPos<BITS>::s(r) == 0 ? 1.0f : (HalfPos<BITS>::s(r) == -24 ? 16777216.0f : 1048576.0f);
}

template <int BITS>
__device__ __forceinline__ void to_halves(const uint32_t (&d)[fw<BITS>() / 2], uint32_t (&hv)[8])
{
    if constexpr (BITS == 8) {
#pragma unroll
        for (int c = 0; c < 4; c++) {
            hv[2 * c] = __builtin_amdgcn_perm(d[c], d[c], 0x0c020c00u);      // bytes 0, 2
            hv[2 * c + 1] = __builtin_amdgcn_perm(d[c], d[c], 0x0c030c01u);  // bytes 1, 3
        }
    } else if constexpr (BITS == 4) {
#pragma unroll
        for (int w = 0; w < 2; w++) {
            const uint32_t p = __builtin_amdgcn_perm(d[w], d[w], 0x0c030c01u);
            hv[4 * w] = d[w] & 0x000f000fu;
            hv[4 * w + 1] = d[w] & 0x00f000f0u;
            hv[4 * w + 2] = p & 0x000f000fu;
            hv[4 * w + 3] = p & 0x00f000f0u;
        }
    } else if constexpr (BITS == 6) {
        // column c is the 24-bit group at bit 24c of the 96-bit block: rows
        // 0/2 and 1/3 are pairs 12 bits apart, moved to bits 4 and 16
        constexpr uint32_t M = 0x003f03f0u;
        hv[0] = (d[0] << 4) & M;
        hv[1] = (d[0] >> 2) & M;
        hv[2] = __builtin_amdgcn_alignbit(d[1], d[0], 20) & M;
        hv[3] = __builtin_amdgcn_alignbit(d[1], d[0], 26) & M;
        hv[4] = __builtin_amdgcn_alignbit(d[2], d[1], 12) & M;
        hv[5] = __builtin_amdgcn_alignbit(d[2], d[1], 18) & M;
        hv[6] = (d[2] >> 4) & M;
        hv[7] = (d[2] >> 10) & M;
    } else {
#pragma unroll
        for (int w = 0; w < 8; w++) hv[w] = d[w];
    }
#pragma unroll
    for (int w = 0; w < 8; w++) asm volatile("" : "+v"(hv[w]));  // keep the halves opaque
}

__device__ __forceinline__ float half_of(uint32_t x, int sel)
{
    const __half2 hh = __builtin_bit_cast(__half2, x);
    return sel ? __high2float(hh) : __low2float(hh);
}

// ---------------------------------------------------------------- requantization
//
// The updated value arrives as z = S'/s in excess form, less a bias: 1 for
// 4/6-bit codes (so that the conversion's saturation at 0 is the lower bound
// of the symmetric range) and 0 for 8-bit codes (so that its saturation at
// 255 is the upper bound).  v_cvt_pk_u8_f32 rounds half to even and
// saturates to [0, 255]; the bound it cannot enforce is checked on the block's
// largest (4/6-bit) or smallest (8-bit) value, and only a block that crosses
// it, or holds a NaN, is converted again: clamped explicitly, with a NaN
// quotient taken as code 0 (an infinite one saturates like any other).

template <int BITS>
constexpr float kBias = BITS == 8 ? 0.0f : 1.0f;

// NaN-propagating three-way extremes (v_maximum3_f32 / v_minimum3_f32): a NaN
// anywhere makes the result NaN, so that the range check below catches it.
// Written as single instructions so that a block's 16 values reduce in a
// chain of exactly 8 (the compiler otherwise rebalances the chain into a
// tree with operands repeated: 9).
__device__ __forceinline__ float fmax3(float a, float b, float c)
{
    float r;
    asm("v_maximum3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float fmin3(float a, float b, float c)
{
    float r;
    asm("v_minimum3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Encode one block whose values z(e) are produced on demand by zf, one output
// group at a time (a column of 8- or 6-bit codes, two columns of 4-bit
// codes), so that at most eight of them are alive at once.  CLAMP applies the
// range explicitly first.  Returns the block's largest (4/6-bit) or smallest
// (8-bit) value for the range check.
template <int BITS, bool CLAMP, typename ZF>
__device__ __forceinline__ float encode_block(ZF zf, uint32_t (&d)[fw<BITS>() / 2])
{
    auto cl = [](float x) {
        if constexpr (!CLAMP) return x;
        else if constexpr (BITS == 8) return fmaxf(x, 1.0f);
        else return __builtin_amdgcn_fmed3f(x, 0.0f, (float)((1 << BITS) - 2));
    };
    float ext = 0.0f;
    if constexpr (BITS == 8) {
#pragma unroll
        for (int c = 0; c < 4; c++) {
            const float z0 = zf(4 * c), z1 = zf(4 * c + 1), z2 = zf(4 * c + 2), z3 = zf(4 * c + 3);
            uint32_t x = pk_u8(cl(z0), 0, 0u);
            x = pk_u8(cl(z1), 1, x);
            x = pk_u8(cl(z2), 2, x);
            d[c] = pk_u8(cl(z3), 3, x);
            // chain: 1 + 1 for the first column's four values, 2 for each later one
            ext = c == 0 ? fmin3(fmin3(z0, z1, z2), z3, z3) : fmin3(fmin3(ext, z0, z1), z2, z3);
        }
    } else if constexpr (BITS == 4) {
        // even fields into the bytes of one word, odd fields into another,
        // then the nibbles interleaved and the bias of every field added
        // back, both words at once as 64-bit shift-adds (every byte is below
        // 15 here, so nothing carries across a nibble)
        uint32_t ev[2] = {0u, 0u}, od[2] = {0u, 0u};
#pragma unroll
        for (int w = 0; w < 2; w++)
#pragma unroll
            for (int p = 0; p < 4; p++) {
                const float ze = zf(8 * w + 2 * p), zo = zf(8 * w + 2 * p + 1);
                ev[w] = pk_u8(cl(ze), p, ev[w]);
                od[w] = pk_u8(cl(zo), p, od[w]);
                ext = (w == 0 && p == 0) ? fmax3(ze, zo, zo) : fmax3(ext, ze, zo);
            }
        const u32x2 e = {ev[0], ev[1]}, o = {od[0], od[1]};
        const uint64_t bias = 0x1111111111111111ull;
        u32x2 x;
        asm("v_lshl_add_u64 %0, %1, 4, %2" : "=v"(x) : "v"(o), "v"(e));
        asm("v_lshl_add_u64 %0, %1, 0, %2" : "=v"(x) : "v"(x), "s"(bias));
        d[0] = x.x;
        d[1] = x.y;
    } else {
        // four codes of a column -> four bytes (each < 63) -> one 24-bit group
        // f0 | f1 << 6 | f2 << 12 | f3 << 18, as two byte dot products whose
        // accumulator adds back the bias (65 = 1 + 64); the four 3-byte groups
        // are then spliced into three dwords with byte permutes
        uint32_t g[4];
#pragma unroll
        for (int c = 0; c < 4; c++) {
            const float z0 = zf(4 * c), z1 = zf(4 * c + 1), z2 = zf(4 * c + 2), z3 = zf(4 * c + 3);
            uint32_t x = pk_u8(cl(z0), 0, 0u);
            x = pk_u8(cl(z1), 1, x);
            x = pk_u8(cl(z2), 2, x);
            x = pk_u8(cl(z3), 3, x);
            const uint32_t lo12 = __builtin_amdgcn_udot4(x, 0x00004001u, 65u, false);
            const uint32_t hi12 = __builtin_amdgcn_udot4(x, 0x40010000u, 65u, false);
            g[c] = lo12 | (hi12 << 12);
            ext = c == 0 ? fmax3(fmax3(z0, z1, z2), z3, z3) : fmax3(fmax3(ext, z0, z1), z2, z3);
        }
        d[0] = __builtin_amdgcn_perm(g[1], g[0], 0x04020100u);  // g0 bytes 0-2, g1 byte 0
        d[1] = __builtin_amdgcn_perm(g[2], g[1], 0x05040201u);  // g1 bytes 1-2, g2 bytes 0-1
        d[2] = __builtin_amdgcn_perm(g[3], g[2], 0x06050402u);  // g2 byte 2, g3 bytes 0-2
    }
    return ext;
}

// true if the block's extreme (encode_block) calls for the explicit clamp: a
// value beyond the bound the conversion cannot enforce, or a NaN
template <int BITS>
__device__ __forceinline__ bool out_of_range(float ext)
{
    if constexpr (BITS == 8) return !(ext > 0.5f);  // rne(0.5) = 0: the code below -Q
    // biased codes 0 .. 2^b - 2 are valid; rne(2^b - 1.5) = 2^b - 2
    else return !(ext <= (float)((1 << BITS) - 2) + 0.5f);
}

// ---------------------------------------------------------------- d = 128 fused step

// scalar load (one per wavefront) from a wave-uniform address
template <typename U>
__device__ __forceinline__ U sload(const U *p)
{
    return *(const __attribute__((address_space(4))) U *)p;
}

// Address of block m of a thread: the tile's (wave-uniform) base advanced by
// whole 4 KB pages, plus the lane's 32-bit offset, plus an immediate below
// 4 KB, so every load and store takes the scalar-base + 32-bit-offset form.
// The page base is pinned to scalar registers, and the loads and the stores
// each take their own opaque copy of the lane offset, so that the optimizer
// does not fold the page steps into 64-bit per-block vector addresses (which
// it would then keep alive, or spill, between the loads and the stores).
template <uint32_t MSTEP>
__device__ __forceinline__ gbyte *block_ptr(uint8_t *tile, uint32_t lane_off, int m)
{
    constexpr uint32_t PAGE = 4096;
    const uint32_t o = (uint32_t)m * MSTEP;
    gbyte *page = (gbyte *)(tile + o / PAGE * PAGE);
    asm volatile("" : "+s"(page));  // scalar registers, recomputed at each use
    return page + lane_off + o % PAGE;
}

typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

// Store a thread's block at page + off + IMM (scalar base, 32-bit lane
// offset, immediate below 4 KB).  Written out because the compiler gives
// these stores 64-bit vector addresses, one more instruction each.  A store
// has no register results, so no wait depends on it.
template <int BITS, bool NT, int IMM>
__device__ __forceinline__ void store_block_asm(const uint8_t *page, uint32_t off,
                                                const uint32_t (&d)[fw<BITS>() / 2])
{
    static_assert(IMM >= 0 && IMM + 16 < 4096, "immediate offset");
    if constexpr (BITS == 4) {
        const u32x2 x = {d[0], d[1]};
        if constexpr (NT)
            asm volatile("global_store_dwordx2 %0, %1, %2 offset:%3 nt" ::"v"(off), "v"(x), "s"(page), "i"(IMM));
        else
            asm volatile("global_store_dwordx2 %0, %1, %2 offset:%3" ::"v"(off), "v"(x), "s"(page), "i"(IMM));
    } else if constexpr (BITS == 6) {
        const u32x3 x = {d[0], d[1], d[2]};
        if constexpr (NT)
            asm volatile("global_store_dwordx3 %0, %1, %2 offset:%3 nt" ::"v"(off), "v"(x), "s"(page), "i"(IMM));
        else
            asm volatile("global_store_dwordx3 %0, %1, %2 offset:%3" ::"v"(off), "v"(x), "s"(page), "i"(IMM));
    } else {
#pragma unroll
        for (int w = 0; w < fw<BITS>() / 2; w += 4) {
            const u32x4 x = {d[w], d[w + 1], d[w + 2], d[w + 3]};
            if constexpr (NT) {
                if (w == 0)
                    asm volatile("global_store_dwordx4 %0, %1, %2 offset:%3 nt" ::"v"(off), "v"(x), "s"(page), "i"(IMM));
                else
                    asm volatile("global_store_dwordx4 %0, %1, %2 offset:%3 nt" ::"v"(off), "v"(x), "s"(page), "i"(IMM + 16));
            } else {
                if (w == 0)
                    asm volatile("global_store_dwordx4 %0, %1, %2 offset:%3" ::"v"(off), "v"(x), "s"(page), "i"(IMM));
                else
                    asm volatile("global_store_dwordx4 %0, %1, %2 offset:%3" ::"v"(off), "v"(x), "s"(page), "i"(IMM + 16));
            }
        }
    }
}

// f(std::integral_constant<int, m>) for m = 0 .. N - 1, in order
template <typename F, int... Ms>
__device__ __forceinline__ void for_blocks(F &&f, std::integer_sequence<int, Ms...>)
{
    (f(std::integral_constant<int, Ms>{}), ...);
}

__device__ __forceinline__ uint32_t opaque(uint32_t x)
{
    asm volatile("" : "+v"(x));
    return x;
}

// The last two steps of a 64-lane sum after the in-row DPP steps: row 0 is
// added into row 1 and row 2 into row 3, then rows 0-1 into rows 2 and 3, so
// row 3 (lanes 48-63) holds the total.  One instruction each (a lane outside
// the row mask keeps its value).
__device__ __forceinline__ float rows_to_row3(float x)
{
    asm volatile("s_nop 1\n\t"
                 "v_add_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
                 "s_nop 1\n\t"
                 "v_add_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf"
                 : "+v"(x));
    return x;
}

// sum over the 64 lanes of a wave, held by lanes 48-63
__device__ __forceinline__ float wave_sum_row3(float x)
{
    x += dpp<0xb1>(x);   // quad_perm [1,0,3,2]
    x += dpp<0x4e>(x);   // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);  // row_half_mirror: sums of 8
    x += dpp<0x140>(x);  // row_mirror: every lane holds its row's sum
    return rows_to_row3(x);
}

// Shared memory of one fused tile.
struct SmemFused {
    alignas(16) float2 wg[128];        // per-row {w_i 2^-s, g_i 2^-s}, w = k_i r_i, g = q_i r_i
    alignas(16) float a[128];          // per-row beta k_i / r_i
    alignas(16) float red[8][2][128];  // [row group][u, y][column] partial sums
    alignas(16) float b[128];          // per-column (v_j - alpha u_j) / c_j
    alignas(8) float2 vc[128];         // per-column {v_j, c_j}
    alignas(16) float sum[2][4];       // per-wave totals of q.k, sum w, sum g (from lanes 48-63)
};

// Per-key-channel gate: pass 2 takes a per-row gate.  pa[i] = {beta k_i / r_i,
// alpha_i 2^-s, OFF (1 - alpha_i) - bias, 0}.
struct SmemFusedK : SmemFused {
    alignas(16) float4 pa[128];
};

template <int BITS, typename T, bool UPDATE, bool CHG, int TPB, typename SM>
__device__ __forceinline__ void tile128(const StepArgs &a, uint32_t n, uint32_t h, SM &sm)
{
    // TPB threads per tile: RG = TPB / 32 row groups, MB = 32 / RG blocks per thread
    constexpr int RG = TPB / 32, MB = 32 / RG;
    static_assert(TPB == 128 || TPB == 256, "128 or 256 threads per tile");
    using P = HalfPos<BITS>;
    constexpr int W = fw<BITS>() / 2;
    constexpr bool QUANT = BITS <= 8;
    constexpr float OFF = QUANT ? (float)(1 << (BITS - 1)) : 0.0f;
    constexpr float BIAS = QUANT ? kBias<BITS> : 0.0f;
    constexpr uint32_t BLK = 2 * fw<BITS>();   // bytes of one 4x4 block
    constexpr uint32_t MSTEP = RG * 32 * BLK;  // bytes between a thread's blocks
    constexpr bool NT = QUANT;                 // code tiles stream nontemporally (measured faster)

    // the tile's own thread index (a 256-thread workgroup may hold two
    // 128-thread tiles, one per half)
    const int t = threadIdx.x & (TPB - 1);
    const int cb = t & 31, rg = t >> 5, tr = t & 127;
    const size_t nh = (size_t)n * (uint32_t)a.H + h;
    const int32_t slot = sload(a.slot_ids + n);
    uint8_t *tile = a.pool + (uint64_t)slot * a.slab + (uint64_t)sload(a.head_off + h);
    const T *q = reinterpret_cast<const T *>(a.q) + nh * 128;
    const T *k = reinterpret_cast<const T *>(a.k) + nh * 128;
    const T *v = reinterpret_cast<const T *>(a.v) + nh * 128;
    const float *rsc = a.rsc + (size_t)slot * a.rstride + (size_t)h * 128;
    const float *csc = a.csc + (size_t)slot * a.cstride + (size_t)h * 128;

    // the per-row (q, k, r, gate) and per-column (v, c) inputs of thread t
    // are loaded before the tile: vector loads complete in issue order, so
    // the row factors can be formed while the tile is still in flight
    const float alpha = UPDATE && !CHG ? sload(a.alpha + nh) : 1.0f;
    const float beta = UPDATE ? sload(a.beta + nh) : 0.0f;
    // row and column tr (with 256 threads, waves 2 and 3 repeat waves 0 and 1
    // here and write the same values)
    const float qi = ld1(q, tr);
    const float ki = UPDATE ? ld1(k, tr) : 0.0f;
    const float rs = QUANT ? rsc[tr] : 1.0f;
    const float gate = CHG ? a.alpha[nh * 128 + tr] : 1.0f;
    const float vj = UPDATE ? ld1(v, tr) : 0.0f;
    const float cjs = QUANT ? csc[tr] : 1.0f;

    // block (rg + RG m, cb) of the tile; the 64 lanes of a wave cover 64
    // consecutive blocks for every m
    const uint32_t lane_off = opaque((uint32_t)(rg * 32 + cb) * BLK);
    uint32_t d[MB][W];
#pragma unroll
    for (int m = 0; m < MB; m++) load_block<BITS, NT>(block_ptr<MSTEP>(tile, lane_off, m), d[m]);

    // per-row factors; the row's power of two 2^-s is folded in (see HalfPos)
    {
        const float us = (tr & 3) == 0 ? unscale<BITS>(0)
                       : (tr & 3) == 1 ? unscale<BITS>(1)
                       : (tr & 3) == 2 ? unscale<BITS>(2) : unscale<BITS>(3);
        const float wi = ki * rs * gate, gi = qi * rs * gate;
        sm.wg[tr] = make_float2(wi * us, gi * us);
        const float ai = QUANT ? beta * ki * __builtin_amdgcn_rcpf(rs) : beta * ki;
        if constexpr (CHG) sm.pa[tr] = make_float4(ai, gate * us, OFF * (1.0f - gate) - BIAS, 0.0f);
        else if (UPDATE) sm.a[tr] = ai;
        sm.vc[tr] = make_float2(vj, cjs);
        // a non-finite row factor or gate of a step sets the pool's sticky flag
        if (UPDATE && __ballot(!__builtin_isfinite(fabsf(ai) + fabsf(CHG ? gate : alpha))) &&
            (t & 63) == 0)
            a.err[0] = 1;
        const float s0 = wave_sum_row3(qi * ki), s1 = wave_sum_row3(wi), s2 = wave_sum_row3(gi);
        if (t < 128 && (t & 63) == 48)
            *reinterpret_cast<float4 *>(&sm.sum[t >> 6][0]) = make_float4(s0, s1, s2, 0.0f);
    }
    __syncthreads();

    uint32_t hv[MB][8];
#pragma unroll
    for (int m = 0; m < MB; m++) to_halves<BITS>(d[m], hv[m]);

    // The two reductions (pass 1, then the column finalisation) run at a
    // raised wave priority: a tile whose data has arrived gets through its two
    // barriers sooner, while other waves on the SIMD are still waiting for
    // memory.
    __builtin_amdgcn_s_setprio(2);

    // pass 1: partial sums of w_i n_ij and g_i n_ij over this thread's rows
    float pu[4] = {0, 0, 0, 0}, py[4] = {0, 0, 0, 0};
    const float2 *wgp = &sm.wg[4 * rg];
#pragma unroll
    for (int m = 0; m < MB; m++) {
        const float4 f01 = *reinterpret_cast<const float4 *>(wgp + 4 * RG * m);
        const float4 f23 = *reinterpret_cast<const float4 *>(wgp + 4 * RG * m + 2);
        const float wr[4] = {f01.x, f01.z, f23.x, f23.z}, gr[4] = {f01.y, f01.w, f23.y, f23.w};
#pragma unroll
        for (int ri = 0; ri < 4; ri++)
#pragma unroll
            for (int cj = 0; cj < 4; cj++) {
                const int e = 4 * cj + ri;
                const float x = half_of(hv[m][P::k(e)], P::sel(e));
                if (UPDATE) pu[cj] = fmaf(wr[ri], x, pu[cj]);
                py[cj] = fmaf(gr[ri], x, py[cj]);
            }
    }
    if (UPDATE) *reinterpret_cast<float4 *>(&sm.red[rg][0][4 * cb]) = make_float4(pu[0], pu[1], pu[2], pu[3]);
    *reinterpret_cast<float4 *>(&sm.red[rg][1][4 * cb]) = make_float4(py[0], py[1], py[2], py[3]);
    __syncthreads();

    // column finalisation: thread j < 128 owns column j
    if (t < 128) {
        float U = UPDATE ? sm.red[0][0][t] : 0.0f, Y = sm.red[0][1][t];
#pragma unroll
        for (int r = 1; r < RG; r++) {
            if (UPDATE) U += sm.red[r][0][t];
            Y += sm.red[r][1][t];
        }
        const float4 s0 = *reinterpret_cast<const float4 *>(&sm.sum[0][0]);
        const float4 s1 = *reinterpret_cast<const float4 *>(&sm.sum[1][0]);
        const float2 vc = sm.vc[t];
        const float cj = vc.y;
        const float yj = cj * (Y - OFF * (s0.z + s1.z));
        if (!UPDATE) {
            a.o[nh * 128 + t] = yj;
        } else {
            const float uj = cj * (U - OFF * (s0.y + s1.y));
            const float e = vc.x - alpha * uj;
            if (a.o) a.o[nh * 128 + t] = fmaf(alpha, yj, beta * (s0.x + s1.x) * e);
            const float bj = QUANT ? e * __builtin_amdgcn_rcpf(cj) : e;
            sm.b[t] = bj;
            // a non-finite column factor sets the pool's sticky flag
            if (__ballot(!__builtin_isfinite(bj)) && (t & 63) == 0) a.err[0] = 1;
        }
    }
    if (!UPDATE) return;
    __syncthreads();
    __builtin_amdgcn_s_setprio(0);
    const float4 b4 = *reinterpret_cast<const float4 *>(&sm.b[4 * cb]);
    const float b[4] = {b4.x, b4.y, b4.z, b4.w};

    // pass 2: z = alpha n + a_i b_j + OFF (1 - alpha) - bias
    const float C = OFF * (1.0f - alpha) - BIAS;
    const float al[4] = {alpha * unscale<BITS>(0), alpha * unscale<BITS>(1), alpha * unscale<BITS>(2),
                         alpha * unscale<BITS>(3)};
    const float *ap = &sm.a[4 * rg];
    const float4 *pp = nullptr;
    if constexpr (CHG) pp = &sm.pa[4 * rg];

    // z(e) of block m from a thread's halves hh, produced on demand
    auto block_zf = [&](int m, const uint32_t (&hh)[8]) {
        float4 fa;
        if constexpr (!CHG) fa = *reinterpret_cast<const float4 *>(ap + 4 * RG * m);
        return [&, m, fa](int e) -> float {
            const int ri = e & 3, cj = e >> 2;
            const float x = half_of(hh[P::k(e)], P::sel(e));
            if constexpr (CHG) {
                const float4 p = pp[4 * RG * m + ri];
                return fmaf(p.y, x, fmaf(p.x, b[cj], p.z));
            } else {
                const float ar = ri == 0 ? fa.x : ri == 1 ? fa.y : ri == 2 ? fa.z : fa.w;
                return fmaf(al[ri], x, fmaf(ar, b[cj], C));
            }
        };
    };

    // the halves are read again in pass 2: keeping them opaque makes the
    // compiler fold the conversion into v_fma_mix_f32 there too instead of
    // keeping 64 converted floats alive across the reduction
#pragma unroll
    for (int m = 0; m < MB; m++)
#pragma unroll
        for (int w = 0; w < 8; w++) asm volatile("" : "+v"(hv[m][w]));
    const uint32_t st_off = opaque(lane_off);  // the stores' own copy

    bool nf = false;
    for_blocks(
        [&](auto M) {
            constexpr int m = decltype(M)::value;
            const auto zf = block_zf(m, hv[m]);
            uint32_t dn[W];
            if constexpr (QUANT) {
                if (out_of_range<BITS>(encode_block<BITS, false>(zf, dn))) {
                    // rare (lanes whose block crosses the bound or holds a NaN):
                    // clamp explicitly; a NaN quotient becomes code 0
                    encode_block<BITS, true>(
                        [&](int e) {
                            const float x = zf(e);
                            return x != x ? OFF - BIAS : x;
                        },
                        dn);
                }
            } else {
                // FP16 pivot: binary16, half to even; a non-finite value is recorded
#pragma unroll
                for (int w = 0; w < 8; w++) {
                    const float z0 = zf(2 * w), z1 = zf(2 * w + 1);
                    nf |= !__builtin_isfinite(z0) || !__builtin_isfinite(z1);
                    const uint32_t lo = __half_as_ushort(__float2half_rn(z0));
                    const uint32_t hi = __half_as_ushort(__float2half_rn(z1));
                    dn[w] = lo | (hi << 16);
                }
            }
            constexpr uint32_t o = (uint32_t)m * MSTEP;
            store_block_asm<BITS, NT, (int)(o % 4096)>(tile + o / 4096 * 4096, st_off, dn);
        },
        std::make_integer_sequence<int, MB>{});
    if (__ballot(nf) && (t & 63) == 0) a.err[0] = 1;
}

template <typename T, bool UPDATE, bool CHG, int TPB, int WPE>
__global__ __launch_bounds__(TPB) __attribute__((amdgpu_waves_per_eu(WPE, 8))) void k_step128(FusedArgs f)
{
    // tile b is request b / H, head b % H: each XCD walks its part of the pool
    // in memory order, so tiles of every width are interleaved on each CU
    // (VALU-heavy narrow codes overlap with memory-heavy wide tiles).  FP32-
    // and BF16-state heads are skipped here and run in k_step128_wide.
    using SM = typename std::conditional<CHG, SmemFusedK, SmemFused>::type;
    __shared__ SM sm;
    uint32_t n, h;
    if (!xcd_tile((uint32_t)f.a.n_req, (uint32_t)f.a.H, f.a.xm, n, h)) return;
    switch (sload(f.head_bits + h)) {
    case 16: tile128<16, T, UPDATE, CHG, TPB>(f.a, n, h, sm); break;
    case 8: tile128<8, T, UPDATE, CHG, TPB>(f.a, n, h, sm); break;
    case 6: tile128<6, T, UPDATE, CHG, TPB>(f.a, n, h, sm); break;
    case 4: tile128<4, T, UPDATE, CHG, TPB>(f.a, n, h, sm); break;
    default: break;
    }
}

// The same step with two 128-thread tiles per 256-thread workgroup (each half
// runs tile128 on its own tile and shared memory; the halves meet at every
// barrier, and a half with no tile, or an FP32/BF16 head, simply ends).
// Measured on full serving launches: a memory-only copy of the step moves its
// bytes 5-6 % faster with two tiles per workgroup than with one.
template <typename T, bool UPDATE, bool CHG, int WPE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, 8))) void k_step128x2(FusedArgs f)
{
    using SM = typename std::conditional<CHG, SmemFusedK, SmemFused>::type;
    __shared__ SM sm[2];
    const uint32_t half = __builtin_amdgcn_readfirstlane(threadIdx.x >> 7);  // uniform per wave
    uint32_t n, h;
    if (!xcd_tile_pair((uint32_t)f.a.n_req, (uint32_t)f.a.H, f.a.xm, half, n, h)) return;
    switch (sload(f.head_bits + h)) {
    case 16: tile128<16, T, UPDATE, CHG, 128>(f.a, n, h, sm[half]); break;
    case 8: tile128<8, T, UPDATE, CHG, 128>(f.a, n, h, sm[half]); break;
    case 6: tile128<6, T, UPDATE, CHG, 128>(f.a, n, h, sm[half]); break;
    case 4: tile128<4, T, UPDATE, CHG, 128>(f.a, n, h, sm[half]); break;
    default: break;
    }
}

template <int FMT, typename T, bool UPDATE, bool CHG>
__global__ __launch_bounds__(kWideTPB) void k_step128_wide(StepArgs a)
{
    // FP32- or BF16-state heads of a d = 128 pool (a.heads / a.Hc)
    using SM = typename std::conditional<CHG, SmemWideK, SmemWide>::type;
    __shared__ SM sm;
    uint32_t n, hc;
    if (!xcd_tile((uint32_t)a.n_req, (uint32_t)a.Hc, a.xm, n, hc)) return;
    tile128_wide<FMT, T, UPDATE, CHG>(a, (int)n, a.heads[hc], sm);
}

// ---------------------------------------------------------------- any shape
//
// d_k, d_v multiples of 4 and <= 256.  Plain and unhurried: one workgroup per
// tile, thread j owns column j for the reductions (reading fields one by
// one), then threads rewrite whole blocks.

__device__ __forceinline__ uint32_t field_get(const uint8_t *tile, int w, long nidx)
{
    const long bit = nidx * w;
    const long byte = bit >> 3;
    const int sh = (int)(bit & 7);
    const int nb = (sh + w + 7) >> 3;
    uint64_t x = 0;
    for (int b = 0; b < nb; b++) x |= (uint64_t)tile[byte + b] << (8 * b);
    x >>= sh;
    return w == 32 ? (uint32_t)x : (uint32_t)(x & ((1ull << w) - 1));
}

template <int BITS>
__device__ __forceinline__ float field_value(uint32_t f)
{
    // centred value: code q for 4/6/8 bits, the value for 16/32 bits
    if constexpr (BITS <= 8) return (float)((int)f - (1 << (BITS - 1)));
    else if constexpr (BITS == 16) return __half2float(__ushort_as_half((unsigned short)f));
    else if constexpr (BITS == kBF16) return __uint_as_float(f << 16);
    else return __uint_as_float(f);
}

template <int BITS, typename T, bool UPDATE, bool CHG>
__global__ __launch_bounds__(256) void k_tile_any(StepArgs a)
{
    constexpr int W = fw<BITS>() / 2;
    constexpr bool QUANT = BITS <= 8;
    constexpr float OFF = QUANT ? (float)(1 << (BITS - 1)) : 0.0f;
    __shared__ float sW[256], sG[256], sA[256], sB[256], sL[256];
    __shared__ float sQK;

    const int t = threadIdx.x;
    const int dk = a.dk, dv = a.dv;
    const int n = blockIdx.x / a.Hc;
    const int hc = blockIdx.x - n * a.Hc;
    const int h = a.heads[hc];
    const long nh = (long)n * a.H + h;
    const int32_t slot = a.slot_ids[n];
    uint8_t *tile = a.pool + (uint64_t)slot * a.slab + (uint64_t)a.head_off[h];
    const T *q = reinterpret_cast<const T *>(a.q);
    const T *k = reinterpret_cast<const T *>(a.k);
    const T *v = reinterpret_cast<const T *>(a.v);
    const float *rsc = a.rsc + (uint64_t)slot * a.rstride + (uint64_t)h * dk;
    const float *csc = a.csc + (uint64_t)slot * a.cstride + (uint64_t)h * dv;
    // per-channel gate: row i is scaled by alpha_i and the column terms take alpha = 1
    const float alpha = UPDATE && !CHG ? a.alpha[nh] : 1.0f;
    const float beta = UPDATE ? a.beta[nh] : 0.0f;

    for (int i = t; i < dk; i += 256) {
        const float ri = QUANT ? rsc[i] : 1.0f;
        const float ki = UPDATE ? ld1(k, nh * dk + i) : 0.0f;
        const float gate = CHG ? a.alpha[nh * dk + i] : alpha;
        sW[i] = ki * ri * (CHG ? gate : 1.0f);
        sG[i] = ld1(q, nh * dk + i) * ri * (CHG ? gate : 1.0f);
        sA[i] = QUANT ? beta * ki / ri : beta * ki;
        sL[i] = gate;
    }
    if (t == 0) {
        float s = 0.0f;
        for (int i = 0; i < dk; i++) s += ld1(q, nh * dk + i) * (UPDATE ? ld1(k, nh * dk + i) : 0.0f);
        sQK = s;
    }
    __syncthreads();
    for (int j = t; j < dv; j += 256) {
        float U = 0.0f, Y = 0.0f;
        for (int i = 0; i < dk; i++) {
            const long nidx = 16L * ((i >> 2) * (dv >> 2) + (j >> 2)) + 4 * (j & 3) + (i & 3);
            const float x = field_value<BITS>(field_get(tile, fw<BITS>(), nidx));
            U = fmaf(sW[i], x, U);
            Y = fmaf(sG[i], x, Y);
        }
        const float cj = QUANT ? csc[j] : 1.0f;
        const float uj = cj * U, yj = cj * Y;
        if (!UPDATE) {
            a.o[nh * dv + j] = yj;
            continue;
        }
        const float e = ld1(v, nh * dv + j) - alpha * uj;
        if (a.o) a.o[nh * dv + j] = fmaf(alpha, yj, beta * sQK * e);
        sB[j] = QUANT ? e / cj : e;
    }
    if (!UPDATE) return;
    __syncthreads();
    const int nblk = (dk >> 2) * (dv >> 2);
    bool nf = false;
    for (int B = t; B < nblk; B += 256) {
        const int i0 = 4 * (B / (dv >> 2)), j0 = 4 * (B % (dv >> 2));
        uint32_t dd[W];
        const uint32_t *src = reinterpret_cast<const uint32_t *>(tile + (long)B * 2 * fw<BITS>());
#pragma unroll
        for (int w = 0; w < W; w++) dd[w] = src[w];
        float f[16], z[16];
        decode<BITS>(dd, f);
#pragma unroll
        for (int cj = 0; cj < 4; cj++)
#pragma unroll
            for (int ri = 0; ri < 4; ri++) {
                const float g = sL[i0 + ri];
                float x = fmaf(g, f[4 * cj + ri], fmaf(sA[i0 + ri], sB[j0 + cj], OFF * (1.0f - g)));
                nf |= !__builtin_isfinite(x);
                if (QUANT && x != x) x = OFF;  // a NaN becomes code 0
                z[4 * cj + ri] = x;
            }
        encode<BITS>(z, dd);
        uint32_t *dst = reinterpret_cast<uint32_t *>(tile + (long)B * 2 * fw<BITS>());
#pragma unroll
        for (int w = 0; w < W; w++) dst[w] = dd[w];
    }
    if (__ballot(nf) && (t & 63) == 0) atomicOr(a.err, 1);
}

// ---------------------------------------------------------------- store
//
// Quantize fp32 states into tiles: one thread per 4x4 block.  The code is
// clamp(rne(x / s), -Q, Q) with s = fl32(r_i c_j) and a correctly rounded
// fp32 division.

template <int BITS>
__global__ __launch_bounds__(256) void k_store(StepArgs a, long total_blocks)
{
    constexpr int W = fw<BITS>() / 2;
    constexpr bool QUANT = BITS <= 8;
    constexpr float OFF = QUANT ? (float)(1 << (BITS - 1)) : 0.0f;
    const long gid = (long)blockIdx.x * 256 + threadIdx.x;
    if (gid >= total_blocks) return;
    const int dk = a.dk, dv = a.dv;
    const long nblk = (long)(dk >> 2) * (dv >> 2);
    const long tix = gid / nblk;
    const long B = gid - tix * nblk;
    const int n = (int)(tix / a.Hc);
    const int h = a.heads[tix - (long)n * a.Hc];
    const long nh = (long)n * a.H + h;
    const int32_t slot = a.slot_ids[n];
    uint8_t *tile = a.pool + (uint64_t)slot * a.slab + (uint64_t)a.head_off[h];
    const float *rsc = a.rsc + (uint64_t)slot * a.rstride + (uint64_t)h * dk;
    const float *csc = a.csc + (uint64_t)slot * a.cstride + (uint64_t)h * dv;
    const int i0 = 4 * (int)(B / (dv >> 2)), j0 = 4 * (int)(B % (dv >> 2));
    const float *S = a.S + nh * (long)dk * dv;
    float z[16];
    bool nf = false;
#pragma unroll
    for (int cj = 0; cj < 4; cj++)
#pragma unroll
        for (int ri = 0; ri < 4; ri++) {
            const float x = S[(long)(i0 + ri) * dv + j0 + cj];
            if constexpr (QUANT) {
                const float s = rsc[i0 + ri] * csc[j0 + cj];
                // decision on fl32(x / s), ties to even, then the symmetric
                // clamp; a NaN quotient becomes code 0, +-Inf the nearest bound
                const float qt = x / s;
                nf |= !__builtin_isfinite(qt);
                const float qf = qt != qt ? 0.0f : fminf(fmaxf(__builtin_rintf(qt), 1.0f - OFF), OFF - 1.0f);
                z[4 * cj + ri] = qf + OFF;  // integer-valued, exact
            } else {
                nf |= !__builtin_isfinite(x);
                z[4 * cj + ri] = x;
            }
        }
    if (__ballot(nf) && (threadIdx.x & 63) == 0) atomicOr(a.err, 1);
    uint32_t dd[W];
    encode<BITS>(z, dd);
    uint32_t *dst = reinterpret_cast<uint32_t *>(tile + B * 2 * fw<BITS>());
#pragma unroll
    for (int w = 0; w < W; w++) dst[w] = dd[w];
}

// ---------------------------------------------------------------- load
//
// Dequantize tiles into fp32 row-major states: one thread per 4x4 block;
// element value = fl32(q * fl32(r_i c_j)) for codes, the binary16 value for
// pivots, the stored value for FP32 heads.

template <int BITS>
__global__ __launch_bounds__(256) void k_load(StepArgs a, float *S, long total_blocks)
{
    constexpr int W = fw<BITS>() / 2;
    constexpr bool QUANT = BITS <= 8;
    constexpr float OFF = QUANT ? (float)(1 << (BITS - 1)) : 0.0f;
    const long gid = (long)blockIdx.x * 256 + threadIdx.x;
    if (gid >= total_blocks) return;
    const int dk = a.dk, dv = a.dv;
    const long nblk = (long)(dk >> 2) * (dv >> 2);
    const long tix = gid / nblk;
    const long B = gid - tix * nblk;
    const int n = (int)(tix / a.Hc);
    const int h = a.heads[tix - (long)n * a.Hc];
    const long nh = (long)n * a.H + h;
    const int32_t slot = a.slot_ids[n];
    const uint8_t *tile = a.pool + (uint64_t)slot * a.slab + (uint64_t)a.head_off[h];
    const float *rsc = a.rsc + (uint64_t)slot * a.rstride + (uint64_t)h * dk;
    const float *csc = a.csc + (uint64_t)slot * a.cstride + (uint64_t)h * dv;
    const int i0 = 4 * (int)(B / (dv >> 2)), j0 = 4 * (int)(B % (dv >> 2));
    uint32_t dd[W];
    const uint32_t *src = reinterpret_cast<const uint32_t *>(tile + B * 2 * fw<BITS>());
#pragma unroll
    for (int w = 0; w < W; w++) dd[w] = src[w];
    float f[16];
    decode<BITS>(dd, f);
    float *dst = S + nh * (long)dk * dv;
#pragma unroll
    for (int cj = 0; cj < 4; cj++)
#pragma unroll
        for (int ri = 0; ri < 4; ri++) {
            float x = f[4 * cj + ri];
            if constexpr (QUANT) {
                const float s = rsc[i0 + ri] * csc[j0 + cj];
                x = (x - OFF) * s;  // the code is exact; one rounding of q * s
            }
            dst[(long)(i0 + ri) * dv + j0 + cj] = x;
        }
}

// ---------------------------------------------------------------- dispatch

template <int BITS, typename T>
static hipError_t launch_bits(Op op, const StepArgs &a, int32_t n_req, hipStream_t st)
{
    if (op == OP_STORE || op == OP_LOAD) {
        const long total = (long)n_req * a.Hc * (a.dk / 4) * (a.dv / 4);
        const long grid = (total + 255) / 256;
        if (op == OP_STORE)
            hipLaunchKernelGGL((k_store<BITS>), dim3((unsigned)grid), dim3(256), 0, st, a, total);
        else
            hipLaunchKernelGGL((k_load<BITS>), dim3((unsigned)grid), dim3(256), 0, st, a,
                               const_cast<float *>(a.S), total);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((long)n_req * a.Hc));
    if (op == OP_STEP)
        hipLaunchKernelGGL((k_tile_any<BITS, T, true, false>), grid, dim3(256), 0, st, a);
    else if (op == OP_STEP_KDA)
        hipLaunchKernelGGL((k_tile_any<BITS, T, true, true>), grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((k_tile_any<BITS, T, false, false>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_t(Op op, int bits, const StepArgs &a, int32_t n_req, hipStream_t st)
{
    switch (bits) {
    case 4: return launch_bits<4, T>(op, a, n_req, st);
    case 6: return launch_bits<6, T>(op, a, n_req, st);
    case 8: return launch_bits<8, T>(op, a, n_req, st);
    case 16: return launch_bits<16, T>(op, a, n_req, st);
    case 32: return launch_bits<32, T>(op, a, n_req, st);
    case kBF16: return launch_bits<kBF16, T>(op, a, n_req, st);
    default: return hipErrorInvalidValue;
    }
}

template <int FMT, typename T>
static void wide128_t(Op op, const StepArgs &a, dim3 grid, hipStream_t st)
{
    if (op == OP_STEP)
        hipLaunchKernelGGL((k_step128_wide<FMT, T, true, false>), grid, dim3(kWideTPB), 0, st, a);
    else if (op == OP_STEP_KDA)
        hipLaunchKernelGGL((k_step128_wide<FMT, T, true, true>), grid, dim3(kWideTPB), 0, st, a);
    else
        hipLaunchKernelGGL((k_step128_wide<FMT, T, false, false>), grid, dim3(kWideTPB), 0, st, a);
}

hipError_t launch_wide128(Op op, int bits, bool qkv_bf16, const StepArgs &a, int32_t n_req,
                          hipStream_t st)
{
    if (n_req <= 0 || a.Hc <= 0) return hipSuccess;
    StepArgs b = a;
    b.n_req = n_req;
    xcd_magic((uint32_t)a.Hc, b.xm);
    const dim3 grid(xcd_grid((uint32_t)n_req, (uint32_t)a.Hc));
    if (bits == 32) {
        if (qkv_bf16) wide128_t<32, uint16_t>(op, b, grid, st);
        else wide128_t<32, float>(op, b, grid, st);
    } else if (bits == kBF16) {
        if (qkv_bf16) wide128_t<kBF16, uint16_t>(op, b, grid, st);
        else wide128_t<kBF16, float>(op, b, grid, st);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, int TPB, int WPE>
static void fused128_t(Op op, const FusedArgs &f, dim3 grid, hipStream_t st)
{
    if (op == OP_STEP)
        hipLaunchKernelGGL((k_step128<T, true, false, TPB, WPE>), grid, dim3(TPB), 0, st, f);
    else if (op == OP_STEP_KDA)
        hipLaunchKernelGGL((k_step128<T, true, true, TPB, WPE>), grid, dim3(TPB), 0, st, f);
    else
        hipLaunchKernelGGL((k_step128<T, false, false, TPB, WPE>), grid, dim3(TPB), 0, st, f);
}

template <int TPB, int WPE>
static void fused128(Op op, bool qkv_bf16, const FusedArgs &f, dim3 grid, hipStream_t st)
{
    if (qkv_bf16) fused128_t<uint16_t, TPB, WPE>(op, f, grid, st);
    else fused128_t<float, TPB, WPE>(op, f, grid, st);
}

template <typename T>
static void fused128x2_t(Op op, const FusedArgs &f, dim3 grid, hipStream_t st)
{
    if (op == OP_STEP)
        hipLaunchKernelGGL((k_step128x2<T, true, false, 5>), grid, dim3(256), 0, st, f);
    else if (op == OP_STEP_KDA)
        hipLaunchKernelGGL((k_step128x2<T, true, true, 5>), grid, dim3(256), 0, st, f);
    else
        hipLaunchKernelGGL((k_step128x2<T, false, false, 5>), grid, dim3(256), 0, st, f);
}

// tile counts that take the 256-thread launch (four waves per tile); larger
// launches pair two 128-thread tiles per workgroup
constexpr uint32_t kWideTilesMin = 1024, kWideTilesMax = 16384;

hipError_t launch_fused128(Op op, bool qkv_bf16, const FusedArgs &f, uint32_t n_blocks,
                          hipStream_t st)
{
    if (n_blocks == 0) return hipSuccess;
    FusedArgs g = f;
    g.a.n_req = (int32_t)(n_blocks / (uint32_t)f.a.H);
    xcd_magic((uint32_t)f.a.H, g.a.xm);
    const dim3 grid(xcd_grid((uint32_t)g.a.n_req, (uint32_t)f.a.H));
    // two waves per tile, each thread holding eight 4x4 blocks as packed
    // halves, the register budget held to 5 waves per SIMD.  A launch of a
    // few thousand tiles (one model layer's heads, say) is bound by the time
    // one tile takes, not by bandwidth: there four waves per tile (four
    // blocks per thread, 8 waves per SIMD) finish each tile sooner.
    // Measured: 3,360-13,440 tiles 4-7 % faster with 256 threads, 20,160 equal,
    // 40,320 and more 4-5 % slower.
    if (n_blocks >= kWideTilesMax) {
        const dim3 grid2(xcd_grid_pair((uint32_t)g.a.n_req, (uint32_t)f.a.H));
        if (qkv_bf16) fused128x2_t<uint16_t>(op, g, grid2, st);
        else fused128x2_t<float>(op, g, grid2, st);
    } else if (n_blocks >= kWideTilesMin) {
        fused128<256, 8>(op, qkv_bf16, g, grid, st);
    } else {
        fused128<128, 5>(op, qkv_bf16, g, grid, st);
    }
    return hipGetLastError();
}

hipError_t launch(Op op, int bits, bool qkv_bf16, const StepArgs &a, int32_t n_req,
                  hipStream_t stream)
{
    if (n_req <= 0 || a.Hc <= 0) return hipSuccess;
    if (qkv_bf16) return launch_t<uint16_t>(op, bits, a, n_req, stream);
    return launch_t<float>(op, bits, a, n_req, stream);
}

// ---------------------------------------------------------------- slot check
//
// Batch validation, separate from the step: every id in [0, n_slots) and no
// id twice.  Each pool keeps an int32 stamp per slot and, after them, the
// generation of the last check.  A check first advances the generation g
// (one thread, which also clears the flag), then exchanges g into the stamp
// of every id it sees; an id whose old stamp is already g has been seen
// earlier in the same check.  The generation lives in device memory, so a
// captured graph of the two launches stays correct on every replay.  Flags:
// 1 = an id out of range, 2 = an id repeated.

constexpr int32_t kGenMax = 0x7fffffff;

__global__ __launch_bounds__(256) void k_check_begin(int32_t *flag, int32_t *stamps, int32_t *gen,
                                                     int32_t n_clear)
{
    // when the generation would wrap, stamps[0, n_clear) are zeroed first so
    // that no stale stamp can equal a new generation
    __shared__ int32_t wrap;
    if (threadIdx.x == 0) wrap = gen[0] >= kGenMax;
    __syncthreads();
    if (wrap) {
        for (int32_t s = threadIdx.x; s < n_clear; s += 256) stamps[s] = 0;
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        gen[0] = wrap ? 1 : gen[0] + 1;
        flag[0] = 0;
    }
}

__global__ __launch_bounds__(256) void k_check_slots(const int32_t *ids, int32_t n, int32_t n_slots,
                                                     int32_t *stamps, const int32_t *gen,
                                                     int32_t *flag)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int32_t id = ids[i];
    if (id < 0 || id >= n_slots) {
        atomicOr(flag, 1);
        return;
    }
    const int32_t g = gen[0];
    if (atomicExch(stamps + id, g) == g) atomicOr(flag, 2);
}

static hipError_t check_slots(const int32_t *ids, int32_t n, int32_t n_slots, int32_t *stamps,
                              int32_t *gen, int32_t n_clear, int32_t *flag, hipStream_t st)
{
    hipLaunchKernelGGL(k_check_begin, dim3(1), dim3(256), 0, st, flag, stamps, gen, n_clear);
    if (n > 0)
        hipLaunchKernelGGL(k_check_slots, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, ids,
                           n, n_slots, stamps, gen, flag);
    return hipGetLastError();
}

hipError_t launch_check_slots(const int32_t *ids, int32_t n, int32_t n_slots, int32_t *stamps,
                              int32_t *flag, hipStream_t st)
{
    // a pool keeps its generation right after its n_slots stamps
    return check_slots(ids, n, n_slots, stamps, stamps + n_slots, n_slots, flag, st);
}

// ---------------------------------------------------------------- allocation-free slot check
//
// The same check with its stamps and generation in a fixed device array of
// this module instead of a pool's table, for callers that cannot allocate.
// Each GPU holds its own copy of the array (zero at module load) until the
// process ends; its address on the current device is looked up once per
// device with hipGetSymbolAddress, and only that address is handed to the
// kernels.  Calls on one GPU share the array, so calls that overlap in time
// on one GPU race.

static __device__ __align__(256) int32_t scratch[kNoAllocMaxSlots + 64];

constexpr int kMaxDevices = 64;
static int32_t *g_scratch[kMaxDevices];
static std::mutex g_scratch_mu;

hipError_t launch_check_slots_noalloc(const int32_t *ids, int32_t n, int32_t n_slots, int32_t *flag,
                                      hipStream_t st)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int32_t *base;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (!g_scratch[dev]) {
            void *p = nullptr;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            g_scratch[dev] = static_cast<int32_t *>(p);
        }
        base = g_scratch[dev];
    }
    // stamps for every supported slot, then the generation
    return check_slots(ids, n, n_slots, base, base + kNoAllocMaxSlots, kNoAllocMaxSlots, flag, st);
}

}  // namespace sqk
