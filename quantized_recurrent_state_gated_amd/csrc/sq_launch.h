// sq_launch.h -- internal interface between the C-ABI host code (sq_api.hip)
// and the gfx950 kernels (sq_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sqk {

// Everything one launch over one width class needs.  Passed by value.
struct StepArgs {
    uint8_t *pool;             // state buffer base
    uint64_t slab;             // bytes per slot
    const int64_t *head_off;   // [H] tile offset inside a slab
    const int32_t *heads;      // [Hc] head ids of this width class
    int32_t Hc;                // heads in the class
    int32_t H;                 // heads per request
    int32_t dk, dv;
    const int32_t *slot_ids;   // [n_req]
    const float *rsc;          // row factors of slot p, head h: rsc + p * rstride + h * dk
    const float *csc;          // column factors: csc + p * cstride + h * dv
    uint64_t rstride, cstride; // 0 = one set of factors shared by every slot
    const void *q, *k, *v;     // [n_req][H][d]
    const float *alpha;        // [n_req][H]; per-channel gate: [n_req][H][dk]
    const float *beta;         // [n_req][H]
    float *o;                  // [n_req][H][dv] or null
    const float *S;            // store: source, load: destination, [n_req][H][dk][dv]
    int32_t *err;              // the pool's sticky device flag (bit 0: a non-finite value)
    int32_t n_req;             // requests in the batch (set by the launchers that need it)
    uint32_t xm[8];            // reciprocals for the XCD-aware tile order (set by the launchers)
};

// OP_STEP_KDA is the step with a per-key-channel gate (alpha [n_req][H][dk]).
enum Op { OP_STEP = 0, OP_READOUT = 1, OP_STORE = 2, OP_LOAD = 3, OP_STEP_KDA = 4 };

// One launch over every tile of a d_k = d_v = 128 pool: tile b is request
// b / H, head b % H, whose width is head_bits[h].
struct FusedArgs {
    StepArgs a;
    const uint8_t *head_bits;  // [H], device
};

// Enqueue `op` for the n_req x Hc tiles of one width class.  bits in
// {4,6,8,16,32,144}; qkv_bf16 selects the q/k/v element type.  Returns the HIP
// error of the launch.
hipError_t launch(Op op, int bits, bool qkv_bf16, const StepArgs &a, int32_t n_req,
                  hipStream_t stream);

// Step or readout over the FP32 (bits 32) or BF16-state (bits 144) heads
// (a.heads / a.Hc) of a d = 128 pool.
hipError_t launch_wide128(Op op, int bits, bool qkv_bf16, const StepArgs &a, int32_t n_req,
                          hipStream_t stream);

// Step or readout over the 4/6/8/16-bit tiles of a d = 128 pool in one launch.
hipError_t launch_fused128(Op op, bool qkv_bf16, const FusedArgs &f, uint32_t n_blocks,
                          hipStream_t stream);

// Advance the check generation (stamps[n_slots]) and clear *flag, then flag
// slot ids out of [0, n_slots) (bit 0) or repeated (bit 1).  stamps holds
// n_slots + 1 int32, zeroed when the pool is made.
hipError_t launch_check_slots(const int32_t *ids, int32_t n, int32_t n_slots, int32_t *stamps,
                              int32_t *flag, hipStream_t stream);

// The same check with its stamps in the module's own fixed device array
// (no allocation); n_slots must be at most kNoAllocMaxSlots.
constexpr int32_t kNoAllocMaxSlots = 65536;
hipError_t launch_check_slots_noalloc(const int32_t *ids, int32_t n, int32_t n_slots, int32_t *flag,
                                      hipStream_t stream);

}  // namespace sqk
