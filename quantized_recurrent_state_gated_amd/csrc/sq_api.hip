// sq_api.hip -- host side of libsq: argument validation, pool layout, the
// small device table, and kernel dispatch per width class.  See include/sq.h
// for the contract of every entry point.
//
// Sources: [P1] "K1 論文詳解" (k1-news, 2026-10-09), 背景 / 方法;
//          [P5] "线性注意力状态量化难题:Qwen状态池70并发就超模型权重" (aitest123),
//          opening (one resident state per concurrent request), 时间维度
//          (per-head bit widths, FP16 pivots), 空间维度 (row x column factors),
//          直接量化为什么会翻车 (the KDA gate of the second model family).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <new>
#include <vector>

#include "../../include/sq.h"
#include "sq_launch.h"

namespace {

// head_bits values: 4/6/8-bit codes, FP16 pivots, FP32 states, BF16 states
constexpr int kNumClasses = 6;
constexpr int kClasses[kNumClasses] = {4, 6, 8, 16, 32, SQ_BITS_BF16};
constexpr int kClassF32 = 4, kClassBF16 = 5;

int class_index(int bits)
{
    for (int c = 0; c < kNumClasses; c++)
        if (kClasses[c] == bits) return c;
    return -1;
}

int field_width(int bits) { return bits == SQ_BITS_BF16 ? 16 : bits; }

bool shape_ok(int32_t dk, int32_t dv)
{
    return dk >= 4 && dv >= 4 && dk <= 256 && dv <= 256 && dk % 4 == 0 && dv % 4 == 0;
}

uint64_t tile_bytes(int bits, int32_t dk, int32_t dv)
{
    return (uint64_t)dk * (uint64_t)dv * (uint64_t)field_width(bits) / 8;
}

uint64_t align256(uint64_t x) { return (x + 255) / 256 * 256; }

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Validate the per-pool shape; fills offsets and the slab size on success.
int layout(int32_t n_heads, int32_t dk, int32_t dv, const uint8_t *head_bits,
           std::vector<int64_t> *off, uint64_t *slab)
{
    if (n_heads < 1 || !head_bits) return SQ_ERR_INVALID;
    if (!shape_ok(dk, dv)) return SQ_ERR_UNSUPPORTED;
    uint64_t o = 0;
    for (int32_t h = 0; h < n_heads; h++) {
        if (class_index(head_bits[h]) < 0) return SQ_ERR_UNSUPPORTED;
        if (off) off->push_back((int64_t)o);
        o += align256(tile_bytes(head_bits[h], dk, dv));
    }
    *slab = o;
    return SQ_OK;
}

// Debug and kernel-selection switches, read from the environment once per
// pool at sq_pool_alloc.  Returns SQ_ERR_INVALID for an SQ_KERNEL value that
// names no kernel family, so that a misspelt switch is not silently ignored.
int read_switches(bool *check_ids, bool *generic)
{
    const char *c = getenv("SQ_CHECK");
    *check_ids = c && *c && strcmp(c, "0") != 0;
    const char *k = getenv("SQ_KERNEL");
    if (!k || !*k || strcmp(k, "tuned") == 0) {
        *generic = false;
        return SQ_OK;
    }
    if (strcmp(k, "generic") == 0) {
        *generic = true;
        return SQ_OK;
    }
    return SQ_ERR_INVALID;
}

}  // namespace

struct sq_pool {
    int32_t n_slots, n_heads, dk, dv;
    std::vector<uint8_t> bits;
    std::vector<int64_t> off;
    uint64_t slab;
    const float *rsc, *csc;
    int64_t sstride;          // scale_slot_stride (0 = factors shared by every slot)
    uint8_t *state;
    uint64_t state_bytes;
    int device;
    void *dtab;               // device: int64 head_off[H] | int32 heads grouped by class | u8 bits[H]
                              //         | pad to 4 | int32 slot stamps[n_slots] | int32 generation
                              //         | int32 sticky error word
    int64_t *d_off;
    uint8_t *d_bits;
    int32_t *d_stamps;        // sq_check_slots' per-slot stamps + generation, zeroed at alloc
    int32_t *d_err;           // set by the kernels (bit 0: a non-finite updated value), zeroed at alloc
    int32_t *d_heads[kNumClasses];
    int32_t n_class[kNumClasses];
    bool check_ids;           // SQ_CHECK at sq_pool_alloc: slot ids are checked on the host per call
    bool generic;             // SQ_KERNEL=generic at sq_pool_alloc: d = 128 takes the generic kernels
};

extern "C" {

uint64_t sq_pool_bytes(int32_t n_slots, int32_t n_heads, int32_t d_k, int32_t d_v,
                       const uint8_t *head_bits)
{
    uint64_t slab = 0;
    if (n_slots < 1) return 0;
    if (layout(n_heads, d_k, d_v, head_bits, nullptr, &slab) != SQ_OK) return 0;
    if (slab > UINT64_MAX / (uint64_t)n_slots) return 0;  // does not fit in 64 bits
    return slab * (uint64_t)n_slots;
}

static int pool_alloc(const sq_pool_desc *desc, sq_pool **out);

int sq_pool_alloc(const sq_pool_desc *desc, sq_pool **out)
{
    // no C++ exception crosses the ABI: a failed host allocation is SQ_ERR_NOMEM
    try {
        return pool_alloc(desc, out);
    } catch (...) {
        if (out) *out = nullptr;
        return SQ_ERR_NOMEM;
    }
}

static int pool_alloc(const sq_pool_desc *desc, sq_pool **out)
{
    if (!desc || !out) return SQ_ERR_INVALID;
    *out = nullptr;
    const sq_pool_desc &d = *desc;
    if (d.n_slots < 1 || d.n_heads < 1 || !d.head_bits || !d.state) return SQ_ERR_INVALID;
    if (!d.row_scale || !d.col_scale) return SQ_ERR_INVALID;
    if (d.scale_slot_stride != 0 && d.scale_slot_stride < d.n_heads) return SQ_ERR_INVALID;
    if (!aligned(d.state, 256) || !aligned(d.row_scale, 16) || !aligned(d.col_scale, 16))
        return SQ_ERR_INVALID;
    std::vector<int64_t> off;
    uint64_t slab = 0;
    int st = layout(d.n_heads, d.d_k, d.d_v, d.head_bits, &off, &slab);
    if (st != SQ_OK) return st;
    if (slab > UINT64_MAX / (uint64_t)d.n_slots || d.state_bytes < slab * (uint64_t)d.n_slots)
        return SQ_ERR_INVALID;
    bool check_ids = false, generic = false;
    if (int sw = read_switches(&check_ids, &generic)) return sw;

    sq_pool *p = new (std::nothrow) sq_pool();
    if (!p) return SQ_ERR_NOMEM;
    p->check_ids = check_ids;
    p->generic = generic;
    p->n_slots = d.n_slots;
    p->n_heads = d.n_heads;
    p->dk = d.d_k;
    p->dv = d.d_v;
    p->bits.assign(d.head_bits, d.head_bits + d.n_heads);
    p->off = off;
    p->slab = slab;
    p->rsc = d.row_scale;
    p->csc = d.col_scale;
    p->sstride = d.scale_slot_stride;
    p->state = static_cast<uint8_t *>(d.state);
    p->state_bytes = d.state_bytes;

    // host image of the device table: offsets, then head ids grouped by width
    const size_t H = (size_t)d.n_heads;
    const size_t stamps_at = (H * 13 + 3) / 4 * 4;
    std::vector<unsigned char> img(stamps_at + ((size_t)d.n_slots + 2) * 4, 0);
    memcpy(img.data(), off.data(), H * 8);
    int32_t *heads = reinterpret_cast<int32_t *>(img.data() + H * 8);
    size_t pos = 0;
    size_t start[kNumClasses];
    for (int c = 0; c < kNumClasses; c++) {
        start[c] = pos;
        p->n_class[c] = 0;
        for (int32_t h = 0; h < d.n_heads; h++)
            if (d.head_bits[h] == kClasses[c]) {
                heads[pos++] = h;
                p->n_class[c]++;
            }
    }
    memcpy(img.data() + H * 12, d.head_bits, H);
    if (hipGetDevice(&p->device) != hipSuccess) {
        delete p;
        return SQ_ERR_HIP;
    }
    if (hipMalloc(&p->dtab, img.size()) != hipSuccess) {
        p->dtab = nullptr;
        delete p;
        return SQ_ERR_NOMEM;
    }
    if (hipMemcpy(p->dtab, img.data(), img.size(), hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(p->dtab);
        delete p;
        return SQ_ERR_HIP;
    }
    p->d_off = static_cast<int64_t *>(p->dtab);
    int32_t *dheads = reinterpret_cast<int32_t *>(static_cast<unsigned char *>(p->dtab) + H * 8);
    for (int c = 0; c < kNumClasses; c++) p->d_heads[c] = dheads + start[c];
    p->d_bits = static_cast<unsigned char *>(p->dtab) + H * 12;
    p->d_stamps = reinterpret_cast<int32_t *>(static_cast<unsigned char *>(p->dtab) + stamps_at);
    p->d_err = p->d_stamps + d.n_slots + 1;
    *out = p;
    return SQ_OK;
}

void sq_pool_free(sq_pool *pool)
{
    if (!pool) return;
    if (pool->dtab) {
        // free on the pool's own device, then restore the caller's
        int cur = -1;
        const bool switched = hipGetDevice(&cur) == hipSuccess && cur != pool->device &&
                              hipSetDevice(pool->device) == hipSuccess;
        (void)hipFree(pool->dtab);
        if (switched) (void)hipSetDevice(cur);
    }
    delete pool;
}

int sq_pool_tile_offset(const sq_pool *pool, int32_t slot, int32_t head, uint64_t *offset,
                        uint64_t *bytes)
{
    if (!pool || !offset || !bytes) return SQ_ERR_INVALID;
    if (slot < 0 || slot >= pool->n_slots || head < 0 || head >= pool->n_heads)
        return SQ_ERR_INVALID;
    *offset = (uint64_t)slot * pool->slab + (uint64_t)pool->off[head];
    *bytes = tile_bytes(pool->bits[head], pool->dk, pool->dv);
    return SQ_OK;
}

static sqk::StepArgs base_args(const sq_pool *p, const int32_t *slot_ids)
{
    sqk::StepArgs a;
    memset(&a, 0, sizeof(a));
    a.pool = p->state;
    a.slab = p->slab;
    a.head_off = p->d_off;
    a.H = p->n_heads;
    a.dk = p->dk;
    a.dv = p->dv;
    a.slot_ids = slot_ids;
    a.rsc = p->rsc;
    a.csc = p->csc;
    a.rstride = (uint64_t)p->sstride * (uint64_t)p->dk;
    a.cstride = (uint64_t)p->sstride * (uint64_t)p->dv;
    a.err = p->d_err;
    return a;
}

// Work is launched on the current device; the pool's buffers live on the
// device that was current at sq_pool_alloc.
static int check_device(const sq_pool *p)
{
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return SQ_ERR_HIP;
    return cur == p->device ? SQ_OK : SQ_ERR_INVALID;
}

// SQ_CHECK: copy the batch's slot ids to the host (synchronizing the
// caller's stream) and reject an id outside [0, n_slots), or, for calls that
// write the pool, an id that appears twice, before any kernel is enqueued.
static int host_check_ids(const sq_pool *p, const int32_t *ids, int32_t n, bool writes, void *stream)
{
    if (int st = check_device(p)) return st;
    try {
        std::vector<int32_t> h((size_t)n);
        if (hipMemcpyAsync(h.data(), ids, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost,
                           (hipStream_t)stream) != hipSuccess ||
            hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
            return SQ_ERR_HIP;
        std::vector<uint8_t> seen(writes ? (size_t)p->n_slots : 0, 0);
        for (int32_t id : h) {
            if (id < 0 || id >= p->n_slots) return SQ_ERR_INVALID;
            if (writes && seen[(size_t)id]++) return SQ_ERR_INVALID;
        }
    } catch (...) {
        return SQ_ERR_NOMEM;
    }
    return SQ_OK;
}

static int run_classes(const sq_pool *p, sqk::Op op, sqk::StepArgs a, bool bf16, int32_t n_req,
                       void *stream)
{
    if (int st = check_device(p)) return st;
    // every launch must fit a 1-D grid of at most 2^31 - 1 workgroups: one per
    // tile for the step and readout, one per 256 blocks for store and load
    const uint64_t tiles = (uint64_t)n_req * (uint64_t)p->n_heads;
    const uint64_t blocks = tiles * (uint64_t)(p->dk / 4) * (uint64_t)(p->dv / 4);
    // (the d = 128 launches round each request's heads up to a multiple of 8)
    if (tiles + 8 * (uint64_t)n_req > 0x7fffffffu || (blocks + 255) / 256 > 0x7fffffffu)
        return SQ_ERR_UNSUPPORTED;
    // d = 128: one launch over the 4/6/8/16-bit tiles in pool order, plus one
    // per wide class (FP32, BF16 states); otherwise one launch per width
    // class, widest tiles first
    static const int order[kNumClasses] = {kClassF32, kClassBF16, 3, 2, 1, 0};
    const bool step_or_read = op == sqk::OP_STEP || op == sqk::OP_STEP_KDA || op == sqk::OP_READOUT;
    if (step_or_read && p->dk == 128 && p->dv == 128 && !p->generic) {
        const uint64_t total = tiles;
        if (p->n_class[kClassF32] + p->n_class[kClassBF16] < p->n_heads) {  // any 4/6/8/16-bit heads
            sqk::FusedArgs f;
            f.a = a;
            f.head_bits = p->d_bits;
            if (sqk::launch_fused128(op, bf16, f, (uint32_t)total, (hipStream_t)stream) != hipSuccess)
                return SQ_ERR_HIP;
        }
        for (int c : {kClassF32, kClassBF16}) {
            if (p->n_class[c] == 0) continue;
            a.heads = p->d_heads[c];
            a.Hc = p->n_class[c];
            if (sqk::launch_wide128(op, kClasses[c], bf16, a, n_req, (hipStream_t)stream) !=
                hipSuccess)
                return SQ_ERR_HIP;
        }
        return SQ_OK;
    }
    for (int oc = 0; oc < kNumClasses; oc++) {
        const int c = order[oc];
        if (p->n_class[c] == 0) continue;
        a.heads = p->d_heads[c];
        a.Hc = p->n_class[c];
        if (sqk::launch(op, kClasses[c], bf16, a, n_req, (hipStream_t)stream) != hipSuccess)
            return SQ_ERR_HIP;
    }
    return SQ_OK;
}

int sq_pool_store(sq_pool *pool, const int32_t *slot_ids, int32_t n_req, const float *S,
                  void *stream)
{
    if (!pool || n_req < 0) return SQ_ERR_INVALID;
    if (n_req == 0) return SQ_OK;
    if (n_req > pool->n_slots || !slot_ids || !S || !aligned(S, 16)) return SQ_ERR_INVALID;
    if (pool->check_ids)
        if (int st = host_check_ids(pool, slot_ids, n_req, true, stream)) return st;
    sqk::StepArgs a = base_args(pool, slot_ids);
    a.S = S;
    return run_classes(pool, sqk::OP_STORE, a, false, n_req, stream);
}

int sq_pool_load(const sq_pool *pool, const int32_t *slot_ids, int32_t n_req, float *S,
                 void *stream)
{
    if (!pool || n_req < 0) return SQ_ERR_INVALID;
    if (n_req == 0) return SQ_OK;
    if (n_req > pool->n_slots || !slot_ids || !S || !aligned(S, 16)) return SQ_ERR_INVALID;
    if (pool->check_ids)
        if (int st = host_check_ids(pool, slot_ids, n_req, false, stream)) return st;
    sqk::StepArgs a = base_args(pool, slot_ids);
    a.S = S;
    return run_classes(pool, sqk::OP_LOAD, a, false, n_req, stream);
}

int sq_decode_step(sq_pool *pool, const int32_t *slot_ids, int32_t n_req, const void *q,
                   const void *k, const void *v, int32_t qkv_dtype, const float *alpha,
                   const float *beta, float *o, void *stream)
{
    if (!pool || n_req < 0) return SQ_ERR_INVALID;
    if (qkv_dtype != SQ_F32 && qkv_dtype != SQ_BF16) return SQ_ERR_INVALID;
    if (n_req == 0) return SQ_OK;
    if (n_req > pool->n_slots || !slot_ids || !q || !k || !v || !alpha || !beta)
        return SQ_ERR_INVALID;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || (o && !aligned(o, 16)))
        return SQ_ERR_INVALID;
    if (pool->check_ids)
        if (int st = host_check_ids(pool, slot_ids, n_req, true, stream)) return st;
    sqk::StepArgs a = base_args(pool, slot_ids);
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.beta = beta;
    a.o = o;
    return run_classes(pool, sqk::OP_STEP, a, qkv_dtype == SQ_BF16, n_req, stream);
}

int sq_decode_step_kda(sq_pool *pool, const int32_t *slot_ids, int32_t n_req, const void *q,
                       const void *k, const void *v, int32_t qkv_dtype, const float *alpha,
                       const float *beta, float *o, void *stream)
{
    if (!pool || n_req < 0) return SQ_ERR_INVALID;
    if (qkv_dtype != SQ_F32 && qkv_dtype != SQ_BF16) return SQ_ERR_INVALID;
    if (n_req == 0) return SQ_OK;
    if (n_req > pool->n_slots || !slot_ids || !q || !k || !v || !alpha || !beta)
        return SQ_ERR_INVALID;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(alpha, 16) ||
        (o && !aligned(o, 16)))
        return SQ_ERR_INVALID;
    if (pool->check_ids)
        if (int st = host_check_ids(pool, slot_ids, n_req, true, stream)) return st;
    sqk::StepArgs a = base_args(pool, slot_ids);
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.beta = beta;
    a.o = o;
    return run_classes(pool, sqk::OP_STEP_KDA, a, qkv_dtype == SQ_BF16, n_req, stream);
}

int sq_readout(const sq_pool *pool, const int32_t *slot_ids, int32_t n_req, const void *q,
               int32_t q_dtype, float *o, void *stream)
{
    if (!pool || n_req < 0) return SQ_ERR_INVALID;
    if (q_dtype != SQ_F32 && q_dtype != SQ_BF16) return SQ_ERR_INVALID;
    if (n_req == 0) return SQ_OK;
    if (n_req > pool->n_slots || !slot_ids || !q || !o || !aligned(q, 16) || !aligned(o, 16))
        return SQ_ERR_INVALID;
    if (pool->check_ids)
        if (int st = host_check_ids(pool, slot_ids, n_req, false, stream)) return st;
    sqk::StepArgs a = base_args(pool, slot_ids);
    a.q = q;
    a.o = o;
    return run_classes(pool, sqk::OP_READOUT, a, q_dtype == SQ_BF16, n_req, stream);
}

int sq_check_slots(sq_pool *pool, const int32_t *slot_ids, int32_t n_req, int32_t *result,
                   void *stream)
{
    if (!pool || !result || n_req < 0 || (n_req > 0 && !slot_ids) || !aligned(result, 4))
        return SQ_ERR_INVALID;
    if (int st = check_device(pool)) return st;
    if (sqk::launch_check_slots(slot_ids, n_req, pool->n_slots, pool->d_stamps, result,
                                (hipStream_t)stream) != hipSuccess)
        return SQ_ERR_HIP;
    return SQ_OK;
}

int sq_check_slots_noalloc(const int32_t *slot_ids, int32_t n_req, int32_t n_slots, int32_t *result,
                           void *stream)
{
    if (!result || n_req < 0 || n_slots < 1 || (n_req > 0 && !slot_ids) || !aligned(result, 4))
        return SQ_ERR_INVALID;
    static_assert(SQ_CHECK_NOALLOC_MAX_SLOTS == sqk::kNoAllocMaxSlots, "one limit");
    if (n_slots > SQ_CHECK_NOALLOC_MAX_SLOTS) return SQ_ERR_UNSUPPORTED;
    if (sqk::launch_check_slots_noalloc(slot_ids, n_req, n_slots, result, (hipStream_t)stream) !=
        hipSuccess)
        return SQ_ERR_HIP;
    return SQ_OK;
}

int sq_pool_last_device_error(sq_pool *pool, void *stream)
{
    if (!pool) return SQ_ERR_INVALID;
    if (int st = check_device(pool)) return st;
    // wait for the caller's work on the pool, then read and clear the word
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return SQ_ERR_HIP;
    int32_t word = 0;
    if (hipMemcpy(&word, pool->d_err, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess)
        return SQ_ERR_HIP;
    if (word == 0) return SQ_OK;
    const int32_t zero = 0;
    if (hipMemcpy(pool->d_err, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess)
        return SQ_ERR_HIP;
    return SQ_ERR_DEVICE;
}

const char *sq_status_string(int status)
{
    switch (status) {
    case SQ_OK: return "ok";
    case SQ_ERR_INVALID: return "invalid argument";
    case SQ_ERR_UNSUPPORTED: return "unsupported bit width or shape";
    case SQ_ERR_HIP: return "HIP runtime error";
    case SQ_ERR_NOMEM: return "out of memory";
    case SQ_ERR_DEVICE: return "a kernel met a non-finite value (NaN or infinity)";
    default: return "unknown status";
    }
}

}  // extern "C"
