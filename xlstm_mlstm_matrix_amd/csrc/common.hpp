// common.hpp -- internal types and device helpers of the gfx950 mLSTM library.
// Not part of the public ABI (that is include/mlstm.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlstm {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// e^x through the hardware base-2 exponential: e^x = 2^(x * log2(e)).
__device__ __forceinline__ float exp_e(float x) {
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// logistic function 1 / (1 + e^{-x}); saturates to exactly 0 or 1, no NaN.
__device__ __forceinline__ float sigmoid(float x) {
    return 1.0f / (1.0f + exp_e(-x));
}

// I/O element <-> float.  bf16 -> float is exact; float -> bf16 rounds to
// nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }

// Where the input rows of a chunkwise call lie: the row of token t of pair p
// starts (p / pdiv) * s_hi + (p % pdiv) * s_lo + t * ld elements from the base
// pointer.  Dense [BH, T, d] rows are pdiv = 1, s_hi = T * d, s_lo = 0, ld = d.
// Only the 64-token role-split kernel (mlstm_ws_kernel) reads other layouts;
// the public entry points pass dense ones.
struct RowLayout {
    long long s_hi, s_lo;
    int ld, pdiv;
};
__host__ __device__ inline RowLayout dense_rows(int T, int d) { return RowLayout{(long long)T * d, 0, d, 1}; }
__host__ __device__ inline long long row_base(const RowLayout &l, int p) {
    return (long long)(p / l.pdiv) * l.s_hi + (long long)(p % l.pdiv) * l.s_lo;
}

// Arguments of the chunkwise forward kernels (one struct, passed by value).
struct FwdArgs {
    const void *q, *k, *v;         // [BH, T, d_qk] x2, [BH, T, d_v]   io dtype
    const float *ig, *fg;          // [BH, T]
    const void *o;                 // [BH, T, d_v]                     io dtype
    const float *C0, *n0, *m0;     // initial state (segment 0), NULL = zero
    void *h;                       // [BH, T, d_v]                     io dtype
    float *CT, *nT, *mT;           // final state, NULL = not wanted
    const float *seg_in;           // incoming state per segment (segmented schedule) or NULL
    float *seg_out;                // local state per segment (state-only pass) or NULL
    int BH, T, dk, dv;
    int seg_len;                   // tokens per segment (multiple of the chunk), T if one segment
    int nseg;                      // segments per sequence
    int ntile;                     // value-column tiles per sequence
    int nseg_out;                  // segments whose local state is produced (state-only pass)
    RowLayout lq, lv;              // rows of q and k; of v and o (role-split kernel only)
};

// Layout of one segment state record in the workspace (float32):
//   C' [d_qk][d_v], n' [d_qk], m, g (sum of log forget gates over the segment)
__host__ __device__ inline size_t seg_state_floats(int dk, int dv) {
    return (size_t)dk * dv + dk + 2;
}

struct StepArgs {
    const void *q, *k, *v;         // [BH, d_qk] x2, [BH, d_v]
    const float *ig, *fg;          // [BH]
    const void *o;                 // [BH, d_v]
    const float *C_in, *n_in, *m_in;
    void *h;
    float *C_out, *n_out, *m_out;
    int BH, dk, dv;
    // row split (nb > 1): workgroup (pair, block) owns rows [block*rows,
    // min(dk, (block+1)*rows)); partial read-outs go to part [BH][nb][dv + 4]
    int nb, rows;
    float *part;
};

// Arguments of the backward kernels.
struct BwdArgs {
    const void *q, *k, *v;         // [BH, T, d_qk] x2, [BH, T, d_v]   io dtype
    const float *ig, *fg;          // [BH, T]
    const void *o;                 // [BH, T, d_v]                     io dtype
    const float *C0, *n0, *m0;     // initial state, NULL = zero
    const void *dh;                // [BH, T, d_v]                     io dtype
    float *gq, *gk, *gv;           // gradients of q, k [BH, T, d_qk], v [BH, T, d_v]
    float *gi, *gf;                // of i~, f~ [BH, T]
    float *go;                     // of o~ [BH, T, d_v]
    float *gC0, *gn0, *gm0;        // of the initial state, NULL = not wanted
    float *ckpt;                   // workspace: state at every chunk start
    int BH, T, dk, dv;
};

// Tokens per chunk and largest head dimensions of the backward kernels.
constexpr int kBwdChunk = 32;
constexpr int kBwdMaxDk = 256, kBwdMaxDv = 512;
// Workspace of one pair, in floats from the pair's base; every section starts
// 16-byte aligned.  Per chunk c: the state at its start (C', n', m; padded so
// that its rows are read with 16-byte loads), the rows a_i = dh sigmoid(o~)/den,
// the matrices P and P~, the scalars (sv, w, beta; dec), the carried gradients
// entering it (G*, g*) and the sum over its tokens of q.dq - k.dk; then one
// dm0 partial per block of value columns and the checkpoint pass's K, V tiles.
struct BwdLayout {
    size_t nch, rec, grec;
    size_t off_a, off_p, off_s, off_g, off_x, off_m, off_tile, total;
};
__host__ __device__ inline BwdLayout bwd_layout(int T, int dk, int dv) {
    const size_t L = kBwdChunk;
    BwdLayout o;
    o.nch = ((size_t)T + L - 1) / L;
    o.rec = ((size_t)dk * dv + dk + 1 + 3) / 4 * 4;
    o.grec = ((size_t)dk * dv + dk + 3) / 4 * 4;
    o.off_a = o.nch * o.rec;
    o.off_p = o.off_a + o.nch * L * dv;
    o.off_s = o.off_p + o.nch * 2 * L * L;
    o.off_g = o.off_s + o.nch * 4 * L;
    o.off_x = o.off_g + o.nch * o.grec;
    o.off_m = o.off_x + (o.nch + 3) / 4 * 4;
    o.off_tile = o.off_m + 64;
    o.total = o.off_tile + L * ((size_t)dk + dv);
    return o;
}
__host__ __device__ inline size_t bwd_ckpt_floats(int T, int dk, int dv) { return bwd_layout(T, dk, dv).total; }

// Launchers (defined in the .hip files).  Return hipSuccess or the launch error.
hipError_t launch_step(const StepArgs &a, int io_bf16, hipStream_t s);
// rows per block of the step's row split and the workspace it needs (0: no split)
int step_rows_per_block(int dk, int dv);
size_t step_workspace_bytes(size_t BH, int dk, int dv);
// size of the fixed per-device scratch of the no-allocation step, and its
// address on device `dev` (looked up once per device, that device current)
constexpr size_t kStepScratchBytes = (size_t)32 << 20;
hipError_t step_scratch(int dev, float **out);
hipError_t launch_fused(const FwdArgs &a, int io_bf16, int chunk, int state_only, hipStream_t s);
hipError_t launch_seg_combine(const FwdArgs &a, float *ws, hipStream_t s);
hipError_t launch_bwd(const BwdArgs &a, int io_bf16, hipStream_t s);

// Tiling choices shared by the planner and the launchers.
int prefill_dkp(int dk);                 // d_qk padded to the kernel's compile-time width
int prefill_bv(int io_bf16, int dk, int dv, int chunk);  // value columns per workgroup
bool prefill_supported(int io_bf16, int dk, int dv, int chunk);  // tiles fit in LDS
// chunk the kernels run with when the caller allows up to `chunk` tokens per
// chunk: the largest of chunk, chunk/2, ..., 16 whose tiles fit (0: none)
int prefill_kernel_chunk(int io_bf16, int dk, int dv, int chunk);
// true when launch_fused runs the role-split kernel for this kernel chunk (the
// only one that reads non-dense row layouts)
bool ws_kernel_selected(int io_bf16, int dk, int dv, int chunk);

}  // namespace mlstm
