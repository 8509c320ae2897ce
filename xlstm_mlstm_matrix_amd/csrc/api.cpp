// api.cpp -- the C ABI of include/mlstm.h: validation, planning, launches.
//
// Every check here runs on the host before any device work, so an invalid
// call enqueues nothing and touches no device.  The library allocates
// nothing and never synchronizes; launches go to the caller's stream.  (The
// one piece of device memory it owns is the fixed scratch array of
// mlstm_step_noalloc, part of its code object, in step.hip.)
#include "mlstm.h"

#include <stdint.h>

#include "common.hpp"
#include "hostcheck.hpp"

using namespace mlstm;

namespace {

const char *kStatus[] = {
    "MLSTM_OK",
    "MLSTM_ERR_NULL: a required pointer is NULL",
    "MLSTM_ERR_SHAPE: a size is not positive or the tensor sizes overflow",
    "MLSTM_ERR_UNSUPPORTED: d_qk, d_v, chunk or dtype outside what the kernels implement",
    "MLSTM_ERR_STATE_ARGS: a state triple was given only in part",
    "MLSTM_ERR_WORKSPACE: workspace missing or smaller than the queried size",
    "MLSTM_ERR_ALIAS: buffers overlap in a way this call does not allow",
    "MLSTM_ERR_HIP: the HIP runtime reported an error",
    "MLSTM_ERR_ALIGN: a pointer is not 16-byte aligned",
    "MLSTM_ERR_BLAS: a hipBLASLt call failed",
    "MLSTM_ERR_SCRATCH: the shape needs more than the fixed per-device scratch of "
    "mlstm_step_noalloc (MLSTM_STEP_NOALLOC_MAX_BYTES); use mlstm_step with a workspace",
};
static_assert(MLSTM_STEP_NOALLOC_MAX_BYTES == kStepScratchBytes, "scratch size out of step");

constexpr int kMaxDk = 256, kMaxDv = 512;
constexpr int kTargetWorkgroups = 256;  // one workgroup per compute unit of an MI355X


bool dims_ok(int dk, int dv) {
    return dk >= 16 && dk <= kMaxDk && dk % 16 == 0 && dv >= 16 && dv <= kMaxDv && dv % 16 == 0;
}
bool chunk_ok(int c) { return c == 16 || c == 32 || c == 64 || c == 128; }

// Schedule of one chunkwise call.
struct Plan {
    int variant;     // MLSTM_VARIANT_FUSED or MLSTM_VARIANT_SEGSCAN
    int kchunk;      // tokens per chunk in the kernels (<= the requested chunk)
    int ntile;       // value-column tiles per sequence
    int nseg;        // segments per sequence
    int seg_len;     // tokens per segment (multiple of chunk)
    size_t ws_state; // floats: copy of n0/m0 for in-place calls (both variants)
    size_t ws_seg;   // floats: segment states (segmented schedule)
    size_t bytes() const { return (ws_state + ws_seg) * sizeof(float); }
};

mlstm_status_t make_plan(int B, int H, int T, int dk, int dv, int chunk, mlstm_dtype_t io,
                         mlstm_variant_t variant, Plan *p) {
    if (B <= 0 || H <= 0 || T <= 0 || dk <= 0 || dv <= 0) return MLSTM_ERR_SHAPE;
    if (io != MLSTM_F32 && io != MLSTM_BF16) return MLSTM_ERR_UNSUPPORTED;
    if (!dims_ok(dk, dv) || !chunk_ok(chunk)) return MLSTM_ERR_UNSUPPORTED;
    if (variant != MLSTM_VARIANT_AUTO && variant != MLSTM_VARIANT_FUSED &&
        variant != MLSTM_VARIANT_SEGSCAN)
        return MLSTM_ERR_UNSUPPORTED;
    const int bf = io == MLSTM_BF16;
    // the chunkwise form is exact for any chunk length: where the requested
    // chunk's tiles do not fit in LDS, a shorter power of two is used
    const int kc = prefill_kernel_chunk(bf, dk, dv, chunk);
    if (kc == 0) return MLSTM_ERR_UNSUPPORTED;
    p->kchunk = kc;
    chunk = kc;
    size_t BH, el;
    if (!mul_ok((size_t)B, (size_t)H, &BH) || BH > (size_t)INT32_MAX / 4) return MLSTM_ERR_SHAPE;
    if (!mul_ok(BH * (size_t)T, (size_t)(dk > dv ? dk : dv), &el) || el > SIZE_MAX / 8)
        return MLSTM_ERR_SHAPE;

    const int bv = prefill_bv(bf, dk, dv, chunk);
    p->ntile = (dv + bv - 1) / bv;
    const long wgs = (long)BH * p->ntile;
    const int nchunks = (T + chunk - 1) / chunk;
    int v = variant;
    if (v == MLSTM_VARIANT_AUTO)
        v = (wgs * 2 <= kTargetWorkgroups && nchunks >= 4) ? MLSTM_VARIANT_SEGSCAN : MLSTM_VARIANT_FUSED;
    p->variant = v;
    p->nseg = 1;
    p->seg_len = T;
    if (v == MLSTM_VARIANT_SEGSCAN) {
        // enough segments to give every compute unit a workgroup, each at
        // least 2 chunks long
        long want = (kTargetWorkgroups + wgs - 1) / wgs;
        if (want < 2) want = 2;
        long maxseg = nchunks / 2;
        if (maxseg < 1) maxseg = 1;
        if (want > maxseg) want = maxseg;
        const int cps = (int)((nchunks + want - 1) / want);  // chunks per segment
        p->seg_len = cps * chunk;
        p->nseg = (T + p->seg_len - 1) / p->seg_len;
    }
    p->ws_state = (BH * (size_t)(dk + 1) + 63) / 64 * 64;
    p->ws_seg = p->nseg > 1 ? BH * (size_t)(2 * p->nseg - 1) * seg_state_floats(dk, dv) : 0;
    return MLSTM_OK;
}

hipError_t copy_async(void *dst, const void *src, size_t bytes, hipStream_t s) {
    return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s);
}

}  // namespace

extern "C" {

const char *mlstm_status_string(mlstm_status_t s) {
    int i = (int)s;
    if (i < 0 || i >= (int)(sizeof(kStatus) / sizeof(kStatus[0]))) return "MLSTM: unknown status";
    return kStatus[i];
}

const char *mlstm_version(void) { return "mlstm-gfx950 0.1.0"; }

mlstm_status_t mlstm_fwd_chunkwise_workspace_size_variant(int B, int H, int T, int d_qk, int d_v,
                                                          int chunk, mlstm_dtype_t io,
                                                          mlstm_variant_t variant, size_t *bytes) {
    if (!bytes) return MLSTM_ERR_NULL;
    Plan p;
    mlstm_status_t st = make_plan(B, H, T, d_qk, d_v, chunk, io, variant, &p);
    if (st != MLSTM_OK) return st;
    *bytes = p.bytes();
    return MLSTM_OK;
}

mlstm_status_t mlstm_fwd_chunkwise_schedule(int B, int H, int T, int d_qk, int d_v, int chunk,
                                            mlstm_dtype_t io, mlstm_variant_t variant,
                                            int *kernel_chunk, int *segments) {
    if (!kernel_chunk || !segments) return MLSTM_ERR_NULL;
    Plan p;
    mlstm_status_t st = make_plan(B, H, T, d_qk, d_v, chunk, io, variant, &p);
    if (st != MLSTM_OK) return st;
    *kernel_chunk = p.kchunk;
    *segments = p.nseg;
    return MLSTM_OK;
}

mlstm_status_t mlstm_fwd_chunkwise_workspace_size(int B, int H, int T, int d_qk, int d_v, int chunk,
                                                  mlstm_dtype_t io, size_t *bytes) {
    return mlstm_fwd_chunkwise_workspace_size_variant(B, H, T, d_qk, d_v, chunk, io,
                                                      MLSTM_VARIANT_AUTO, bytes);
}

}  // extern "C"

namespace mlstm {

// The chunkwise forward with the rows of q, k (lq) and of v, o~ (lv) in the
// given layouts, NULL for dense.  Non-dense layouts are for callers inside the
// library whose buffers hold B*H*T rows of each input in a strided order (the
// layer's all-heads projections); they need the role-split kernel
// (MLSTM_ERR_UNSUPPORTED otherwise).  The byte ranges checked for overlap are
// B*H*T*d elements from each base, as for dense inputs.
mlstm_status_t fwd_chunkwise_rows(const void *q, const void *k, const void *v, const float *i_pre,
                                  const float *f_pre, const void *o_pre, const float *C0,
                                  const float *n0, const float *m0, void *h, float *C_T, float *n_T,
                                  float *m_T, int B, int H, int T, int d_qk, int d_v, int chunk,
                                  mlstm_dtype_t io, mlstm_variant_t variant, void *workspace,
                                  size_t workspace_bytes, void *stream, const RowLayout *lq,
                                  const RowLayout *lv) {
    if (!q || !k || !v || !i_pre || !f_pre || !o_pre || !h) return MLSTM_ERR_NULL;
    Plan p;
    mlstm_status_t st = make_plan(B, H, T, d_qk, d_v, chunk, io, variant, &p);
    if (st != MLSTM_OK) return st;
    if ((lq || lv) && !ws_kernel_selected(io == MLSTM_BF16, d_qk, d_v, p.kchunk)) return MLSTM_ERR_UNSUPPORTED;
    const int in0 = (C0 != nullptr) + (n0 != nullptr) + (m0 != nullptr);
    const int out0 = (C_T != nullptr) + (n_T != nullptr) + (m_T != nullptr);
    if ((in0 != 0 && in0 != 3) || (out0 != 0 && out0 != 3)) return MLSTM_ERR_STATE_ARGS;
    if (!all_aligned({q, k, v, i_pre, f_pre, o_pre, C0, n0, m0, h, C_T, n_T, m_T, workspace}))
        return MLSTM_ERR_ALIGN;

    const size_t es = io == MLSTM_BF16 ? 2 : 4;
    const size_t BH = (size_t)B * H;
    const size_t nqk = BH * T * d_qk, nv = BH * T * d_v, ng = BH * T;
    const size_t nC = BH * d_qk * d_v, nn = BH * d_qk, nm = BH;
    const Range rq = rng(q, nqk * es), rk = rng(k, nqk * es), rv = rng(v, nv * es);
    const Range ri = rng(i_pre, ng * 4), rf = rng(f_pre, ng * 4), ro = rng(o_pre, nv * es);
    const Range rC0 = rng(C0, nC * 4), rn0 = rng(n0, nn * 4), rm0 = rng(m0, nm * 4);
    const Range rh = rng(h, nv * es);
    const Range rCT = rng(C_T, nC * 4), rnT = rng(n_T, nn * 4), rmT = rng(m_T, nm * 4);
    const Range inputs[] = {rq, rk, rv, ri, rf, ro, rC0, rn0, rm0};
    const Range outs[] = {rh, rCT, rnT, rmT};
    // an output may coincide exactly with its own initial-state buffer, and
    // overlap nothing else
    for (int o = 0; o < 4; ++o) {
        for (int i = 0; i < 9; ++i) {
            const bool allowed = (o == 1 && i == 6) || (o == 2 && i == 7) || (o == 3 && i == 8);
            if (overlaps(outs[o], inputs[i]) && !(allowed && same(outs[o], inputs[i])))
                return MLSTM_ERR_ALIAS;
        }
        for (int o2 = o + 1; o2 < 4; ++o2)
            if (overlaps(outs[o], outs[o2])) return MLSTM_ERR_ALIAS;
    }
    const size_t need = p.bytes();
    if (need > 0 && (!workspace || workspace_bytes < need)) return MLSTM_ERR_WORKSPACE;
    const Range rws = rng(workspace, need);
    for (const Range &r : inputs)
        if (overlaps(rws, r)) return MLSTM_ERR_ALIAS;
    for (const Range &r : outs)
        if (overlaps(rws, r)) return MLSTM_ERR_ALIAS;

    hipStream_t s = static_cast<hipStream_t>(stream);
    FwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.ig = i_pre; a.fg = f_pre; a.o = o_pre;
    a.C0 = C0; a.n0 = n0; a.m0 = m0;
    a.h = h; a.CT = C_T; a.nT = n_T; a.mT = m_T;
    a.BH = (int)BH; a.T = T; a.dk = d_qk; a.dv = d_v;
    a.ntile = p.ntile; a.nseg = p.nseg; a.seg_len = p.seg_len;
    a.lq = lq ? *lq : dense_rows(T, d_qk);
    a.lv = lv ? *lv : dense_rows(T, d_v);
    const int bf = io == MLSTM_BF16;
    float *ws = static_cast<float *>(workspace);
    hipError_t e = hipSuccess;

    if (p.nseg == 1) {
        // several column tiles read n0/m0 while one of them writes n_T/m_T:
        // for an in-place call read a copy instead
        if (C0 && (n_T == n0 || m_T == m0) && p.ntile > 1) {
            float *ncopy = ws, *mcopy = ws + nn;
            e = copy_async(ncopy, n0, nn * 4, s);
            if (e == hipSuccess) e = copy_async(mcopy, m0, nm * 4, s);
            a.n0 = ncopy;
            a.m0 = mcopy;
        }
        if (e == hipSuccess) e = launch_fused(a, bf, p.kchunk, 0, s);
    } else {
        float *seg = ws + p.ws_state;
        const size_t rec = seg_state_floats(d_qk, d_v);
        a.seg_out = seg;                                  // local states, segments 0..nseg-2
        e = launch_fused(a, bf, p.kchunk, 1, s);
        if (e == hipSuccess) e = launch_seg_combine(a, seg, s);  // reads C0/n0/m0
        if (e == hipSuccess) {
            a.seg_in = seg + BH * (size_t)(p.nseg - 1) * rec;  // incoming state per segment
            a.seg_out = nullptr;
            e = launch_fused(a, bf, p.kchunk, 0, s);
        }
    }
    return e == hipSuccess ? MLSTM_OK : MLSTM_ERR_HIP;
}

}  // namespace mlstm

extern "C" {

mlstm_status_t mlstm_fwd_chunkwise_variant(const void *q, const void *k, const void *v,
                                           const float *i_pre, const float *f_pre,
                                           const void *o_pre, const float *C0, const float *n0,
                                           const float *m0, void *h, float *C_T, float *n_T,
                                           float *m_T, int B, int H, int T, int d_qk, int d_v,
                                           int chunk, mlstm_dtype_t io, mlstm_variant_t variant,
                                           void *workspace, size_t workspace_bytes, void *stream) {
    return fwd_chunkwise_rows(q, k, v, i_pre, f_pre, o_pre, C0, n0, m0, h, C_T, n_T, m_T, B, H, T,
                              d_qk, d_v, chunk, io, variant, workspace, workspace_bytes, stream,
                              nullptr, nullptr);
}

mlstm_status_t mlstm_fwd_chunkwise(const void *q, const void *k, const void *v, const float *i_pre,
                                   const float *f_pre, const void *o_pre, const float *C0,
                                   const float *n0, const float *m0, void *h, float *C_T,
                                   float *n_T, float *m_T, int B, int H, int T, int d_qk, int d_v,
                                   int chunk, mlstm_dtype_t io, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    return mlstm_fwd_chunkwise_variant(q, k, v, i_pre, f_pre, o_pre, C0, n0, m0, h, C_T, n_T, m_T,
                                       B, H, T, d_qk, d_v, chunk, io, MLSTM_VARIANT_AUTO, workspace,
                                       workspace_bytes, stream);
}

mlstm_status_t mlstm_step_workspace_size(int B, int H, int d_qk, int d_v, mlstm_dtype_t io,
                                         size_t *bytes) {
    if (!bytes) return MLSTM_ERR_NULL;
    *bytes = 0;
    if (B <= 0 || H <= 0 || d_qk <= 0 || d_v <= 0) return MLSTM_ERR_SHAPE;
    if (io != MLSTM_F32 && io != MLSTM_BF16) return MLSTM_ERR_UNSUPPORTED;
    if (!dims_ok(d_qk, d_v)) return MLSTM_ERR_UNSUPPORTED;
    size_t BH;
    if (!mul_ok((size_t)B, (size_t)H, &BH) || BH > (size_t)INT32_MAX) return MLSTM_ERR_SHAPE;
    *bytes = step_workspace_bytes(BH, d_qk, d_v);
    return MLSTM_OK;
}

}  // extern "C"

namespace {

// mlstm_step and mlstm_step_noalloc: the same checks and launches; the second
// takes the row split's workspace from the library's fixed per-device scratch
// (after every host-side check, so an invalid call touches no device).
mlstm_status_t step_call(const void *q, const void *k, const void *v, const float *i_pre,
                         const float *f_pre, const void *o_pre, const float *C_in,
                         const float *n_in, const float *m_in, void *h, float *C_out,
                         float *n_out, float *m_out, int B, int H, int d_qk, int d_v,
                         mlstm_dtype_t io, void *workspace, size_t workspace_bytes,
                         bool fixed_scratch, void *stream) {
    if (!q || !k || !v || !i_pre || !f_pre || !o_pre || !h || !C_out || !n_out || !m_out)
        return MLSTM_ERR_NULL;
    if (B <= 0 || H <= 0 || d_qk <= 0 || d_v <= 0) return MLSTM_ERR_SHAPE;
    if (io != MLSTM_F32 && io != MLSTM_BF16) return MLSTM_ERR_UNSUPPORTED;
    if (!dims_ok(d_qk, d_v)) return MLSTM_ERR_UNSUPPORTED;
    size_t BH;
    if (!mul_ok((size_t)B, (size_t)H, &BH) || BH > (size_t)INT32_MAX) return MLSTM_ERR_SHAPE;
    const int in0 = (C_in != nullptr) + (n_in != nullptr) + (m_in != nullptr);
    if (in0 != 0 && in0 != 3) return MLSTM_ERR_STATE_ARGS;
    if (!all_aligned({q, k, v, i_pre, f_pre, o_pre, C_in, n_in, m_in, h, C_out, n_out, m_out,
                      workspace}))
        return MLSTM_ERR_ALIGN;

    const size_t es = io == MLSTM_BF16 ? 2 : 4;
    const size_t nC = BH * d_qk * d_v, nn = BH * d_qk;
    const Range inputs[] = {rng(q, BH * d_qk * es), rng(k, BH * d_qk * es), rng(v, BH * d_v * es),
                            rng(i_pre, BH * 4),      rng(f_pre, BH * 4),      rng(o_pre, BH * d_v * es),
                            rng(C_in, nC * 4),       rng(n_in, nn * 4),       rng(m_in, BH * 4)};
    const Range outs[] = {rng(h, BH * d_v * es), rng(C_out, nC * 4), rng(n_out, nn * 4),
                          rng(m_out, BH * 4)};
    for (int o = 0; o < 4; ++o) {
        for (int i = 0; i < 9; ++i) {
            const bool allowed = (o == 1 && i == 6) || (o == 2 && i == 7) || (o == 3 && i == 8);
            if (overlaps(outs[o], inputs[i]) && !(allowed && same(outs[o], inputs[i])))
                return MLSTM_ERR_ALIAS;
        }
        for (int o2 = o + 1; o2 < 4; ++o2)
            if (overlaps(outs[o], outs[o2])) return MLSTM_ERR_ALIAS;
    }

    StepArgs a{};
    a.q = q; a.k = k; a.v = v; a.ig = i_pre; a.fg = f_pre; a.o = o_pre;
    a.C_in = C_in; a.n_in = n_in; a.m_in = m_in;
    a.h = h; a.C_out = C_out; a.n_out = n_out; a.m_out = m_out;
    a.BH = (int)BH; a.dk = d_qk; a.dv = d_v;
    a.nb = 1; a.rows = d_qk;
    // with a workspace, large memories are split into row blocks (one
    // workgroup each); without one, one workgroup streams each pair
    const size_t need = step_workspace_bytes(BH, d_qk, d_v);
    if (fixed_scratch) {
        if (need > kStepScratchBytes) return MLSTM_ERR_SCRATCH;
        workspace = nullptr;
        if (need > 0) {
            int dev = 0;
            float *p = nullptr;
            if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) != hipSuccess ||
                step_scratch(dev, &p) != hipSuccess)
                return MLSTM_ERR_HIP;
            workspace = p;
            workspace_bytes = kStepScratchBytes;
        }
    }
    if (workspace && need > 0) {
        if (workspace_bytes < need) return MLSTM_ERR_WORKSPACE;
        const Range rws = rng(workspace, need);
        for (const Range &r : inputs)
            if (overlaps(rws, r)) return MLSTM_ERR_ALIAS;
        for (const Range &r : outs)
            if (overlaps(rws, r)) return MLSTM_ERR_ALIAS;
        a.rows = step_rows_per_block(d_qk, d_v);
        a.nb = (d_qk + a.rows - 1) / a.rows;
        if (BH > (size_t)INT32_MAX / (size_t)a.nb) return MLSTM_ERR_SHAPE;
        a.part = static_cast<float *>(workspace);
    }
    hipError_t e = launch_step(a, io == MLSTM_BF16, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MLSTM_OK : MLSTM_ERR_HIP;
}

}  // namespace

extern "C" {

mlstm_status_t mlstm_step(const void *q, const void *k, const void *v, const float *i_pre,
                          const float *f_pre, const void *o_pre, const float *C_in,
                          const float *n_in, const float *m_in, void *h, float *C_out, float *n_out,
                          float *m_out, int B, int H, int d_qk, int d_v, mlstm_dtype_t io,
                          void *workspace, size_t workspace_bytes, void *stream) {
    return step_call(q, k, v, i_pre, f_pre, o_pre, C_in, n_in, m_in, h, C_out, n_out, m_out, B, H,
                     d_qk, d_v, io, workspace, workspace_bytes, false, stream);
}

mlstm_status_t mlstm_step_noalloc(const void *q, const void *k, const void *v, const float *i_pre,
                                  const float *f_pre, const void *o_pre, const float *C_in,
                                  const float *n_in, const float *m_in, void *h, float *C_out,
                                  float *n_out, float *m_out, int B, int H, int d_qk, int d_v,
                                  mlstm_dtype_t io, void *stream) {
    return step_call(q, k, v, i_pre, f_pre, o_pre, C_in, n_in, m_in, h, C_out, n_out, m_out, B, H,
                     d_qk, d_v, io, nullptr, 0, true, stream);
}

// ---- backward

static mlstm_status_t bwd_check_dims(int B, int H, int T, int d_qk, int d_v, int chunk, mlstm_dtype_t io,
                              size_t *bytes) {
    if (B <= 0 || H <= 0 || T <= 0 || d_qk <= 0 || d_v <= 0) return MLSTM_ERR_SHAPE;
    if (io != MLSTM_F32 && io != MLSTM_BF16) return MLSTM_ERR_UNSUPPORTED;
    if (!dims_ok(d_qk, d_v) || d_qk > kBwdMaxDk || d_v > kBwdMaxDv || !chunk_ok(chunk))
        return MLSTM_ERR_UNSUPPORTED;
    size_t BH, n;
    if (!mul_ok((size_t)B, (size_t)H, &BH) || BH > (size_t)INT32_MAX) return MLSTM_ERR_SHAPE;
    if (!mul_ok(BH, (size_t)T, &n) || !mul_ok(n, (size_t)(d_qk > d_v ? d_qk : d_v), &n))
        return MLSTM_ERR_SHAPE;
    // one sequence's q, k, v and gradients are addressed through 32-bit
    // offsets, up to a chunk past T
    if ((size_t)(T + kBwdChunk) * (size_t)(d_qk > d_v ? d_qk : d_v) * sizeof(float) >= ((size_t)1 << 31))
        return MLSTM_ERR_UNSUPPORTED;
    if (!mul_ok(BH, bwd_ckpt_floats(T, d_qk, d_v), &n) || !mul_ok(n, sizeof(float), bytes))
        return MLSTM_ERR_SHAPE;
    return MLSTM_OK;
}

mlstm_status_t mlstm_bwd_chunkwise_workspace_size(int B, int H, int T, int d_qk, int d_v, int chunk,
                                                  mlstm_dtype_t io, size_t *bytes) {
    if (!bytes) return MLSTM_ERR_NULL;
    return bwd_check_dims(B, H, T, d_qk, d_v, chunk, io, bytes);
}

mlstm_status_t mlstm_bwd_chunkwise(const void *q, const void *k, const void *v, const float *i_pre,
                                   const float *f_pre, const void *o_pre, const float *C0,
                                   const float *n0, const float *m0, const void *dh, float *dq,
                                   float *dk, float *dv, float *d_i, float *d_f, float *d_o,
                                   float *dC0, float *dn0, float *dm0, int B, int H, int T, int d_qk,
                                   int d_v, int chunk, mlstm_dtype_t io, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    if (!q || !k || !v || !i_pre || !f_pre || !o_pre || !dh || !dq || !dk || !dv || !d_i || !d_f ||
        !d_o)
        return MLSTM_ERR_NULL;
    size_t need;
    mlstm_status_t st = bwd_check_dims(B, H, T, d_qk, d_v, chunk, io, &need);
    if (st != MLSTM_OK) return st;
    const int in0 = (C0 != nullptr) + (n0 != nullptr) + (m0 != nullptr);
    const int out0 = (dC0 != nullptr) + (dn0 != nullptr) + (dm0 != nullptr);
    if ((in0 != 0 && in0 != 3) || (out0 != 0 && out0 != 3)) return MLSTM_ERR_STATE_ARGS;
    if (!all_aligned({q, k, v, i_pre, f_pre, o_pre, C0, n0, m0, dh, dq, dk, dv, d_i, d_f, d_o, dC0, dn0,
                      dm0, workspace}))
        return MLSTM_ERR_ALIGN;

    const size_t es = io == MLSTM_BF16 ? 2 : 4;
    const size_t BH = (size_t)B * H;
    const size_t nqk = BH * T * d_qk, nv = BH * T * d_v, ng = BH * T;
    const size_t nC = BH * d_qk * d_v, nn = BH * d_qk;
    const Range inputs[] = {rng(q, nqk * es), rng(k, nqk * es), rng(v, nv * es), rng(i_pre, ng * 4),
                            rng(f_pre, ng * 4), rng(o_pre, nv * es), rng(C0, nC * 4), rng(n0, nn * 4),
                            rng(m0, BH * 4), rng(dh, nv * es)};
    const Range outs[] = {rng(dq, nqk * 4), rng(dk, nqk * 4), rng(dv, nv * 4), rng(d_i, ng * 4),
                          rng(d_f, ng * 4), rng(d_o, nv * 4), rng(dC0, nC * 4), rng(dn0, nn * 4),
                          rng(dm0, BH * 4)};
    if (!workspace || workspace_bytes < need) return MLSTM_ERR_WORKSPACE;
    const Range rws = rng(workspace, need);
    for (const Range &o : outs) {
        for (const Range &i : inputs)
            if (overlaps(o, i)) return MLSTM_ERR_ALIAS;
        if (overlaps(o, rws)) return MLSTM_ERR_ALIAS;
    }
    for (size_t o = 0; o < sizeof(outs) / sizeof(outs[0]); ++o)
        for (size_t o2 = o + 1; o2 < sizeof(outs) / sizeof(outs[0]); ++o2)
            if (overlaps(outs[o], outs[o2])) return MLSTM_ERR_ALIAS;
    for (const Range &i : inputs)
        if (overlaps(rws, i)) return MLSTM_ERR_ALIAS;

    BwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.ig = i_pre; a.fg = f_pre; a.o = o_pre;
    a.C0 = C0; a.n0 = n0; a.m0 = m0; a.dh = dh;
    a.gq = dq; a.gk = dk; a.gv = dv; a.gi = d_i; a.gf = d_f; a.go = d_o;
    a.gC0 = dC0; a.gn0 = dn0; a.gm0 = dm0;
    a.ckpt = static_cast<float *>(workspace);
    a.BH = (int)BH; a.T = T; a.dk = d_qk; a.dv = d_v;
    hipError_t e = launch_bwd(a, io == MLSTM_BF16, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MLSTM_OK : MLSTM_ERR_HIP;
}

}  // extern "C"
