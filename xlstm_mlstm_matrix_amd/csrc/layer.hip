// layer.hip -- the mLSTM layer forward: input projections, gates, the cell.
//
// The xLSTM notes' example mLSTM module (section "mLSTM", its listing of the
// recurrent forward) maps each token x_t of width d_model through linear
// layers with bias to the query, key, value and output-gate pre-activation,
// and to one input-gate and one forget-gate pre-activation; the forget one is
// the log of the forget gate in the stabilized recurrence.  Per head h:
//   q = W_q[h] x + b_q[h],  k = W_k[h] x + b_k[h]          (d_qk)
//   v = W_v[h] x + b_v[h],  o~ = W_o[h] x + b_o[h]         (d_v)
//   i~ = W_i[h] . x + b_i[h],  f~ = W_f[h] . x + b_f[h]    (scalars)
// then the chunkwise cell over each (head, batch) cell.
//
// Layout choice: cells are ordered head-major (cell p = h*B + b).
//  * Where the cell runs the 64-token role-split kernel (bf16, the 7B-layer
//    heads), which reads strided input rows, each weight is ONE GEMM over all
//    heads: M = H*d, N = B*T, K = d_model, column-major [H*d, B*T], so token
//    b*T + t holds every head's features in one row of H*d; cell (h, b) reads
//    the head-h part of rows b*T .. b*T + T - 1.  Four wide GEMMs run at a
//    higher fraction of the MFMA peak than 4*H narrow ones (M = d).
//  * Otherwise one head's projection of every token of every batch is one
//    GEMM with M = d, N = B*T and K = d_model, whose column-major result
//    [d, B*T] is exactly the cell's row-major [B, T, d] block of head h.
// Neither needs a permute pass.  The per-feature bias is hipBLASLt's
// bias epilogue (one value per output row).  The gate pre-activations of
// head h are the GEMM [B*T, H] = x W_i^T (column-major, so each head's B*T
// values are contiguous: the cell's gate layout), float32 out; with W_i and
// W_f copied one after the other into the workspace, a single GEMM
// [B*T, 2H] writes both and reads x once.  Their biases are added by a small
// kernel.  The cell is mlstm_fwd_chunkwise with the
// (batch, head) roles of its B and H swapped.
//
// The projections are plain library GEMMs (hipBLASLt, bf16 or fp32 inputs,
// fp32 accumulation).  The library keeps one hipBLASLt handle per device and
// the algorithm it picked per GEMM shape, created on first use.
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "common.hpp"
#include "hostcheck.hpp"
#include "mlstm.h"

namespace mlstm {

// the chunkwise forward with strided input rows (api.cpp)
mlstm_status_t fwd_chunkwise_rows(const void *q, const void *k, const void *v, const float *i_pre,
                                  const float *f_pre, const void *o_pre, const float *C0,
                                  const float *n0, const float *m0, void *h, float *C_T, float *n_T,
                                  float *m_T, int B, int H, int T, int d_qk, int d_v, int chunk,
                                  mlstm_dtype_t io, mlstm_variant_t variant, void *workspace,
                                  size_t workspace_bytes, void *stream, const RowLayout *lq,
                                  const RowLayout *lv);

namespace {

constexpr size_t kGemmWorkspace = size_t(32) << 20;  // hipBLASLt's share of the workspace

__global__ __launch_bounds__(256) void gate_bias_kernel(float *gi, float *gf, const float *bi,
                                                        const float *bf, size_t per_head, int H) {
    const size_t n = per_head * (size_t)H;
    for (size_t x = blockIdx.x * (size_t)blockDim.x + threadIdx.x; x < n;
         x += (size_t)gridDim.x * blockDim.x) {
        const int h = (int)(x / per_head);
        gi[x] += bi[h];
        gf[x] += bf[h];
    }
}

struct AlgoKey {
    int dev, m, n, k, ab, d, bias;
    bool operator<(const AlgoKey &o) const {
        return std::tie(dev, m, n, k, ab, d, bias) < std::tie(o.dev, o.m, o.n, o.k, o.ab, o.d, o.bias);
    }
};

std::mutex g_mu;
std::map<int, hipblasLtHandle_t> g_handle;
std::map<AlgoKey, hipblasLtMatmulAlgo_t> g_algo;

hipblasLtHandle_t handle_for(int dev) {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_handle.find(dev);
    if (it != g_handle.end()) return it->second;
    hipblasLtHandle_t h = nullptr;
    if (hipblasLtCreate(&h) != HIPBLAS_STATUS_SUCCESS) return nullptr;
    g_handle[dev] = h;
    return h;
}

// D (column-major m x n, leading dimension m) = A^T B (+ bias[row]), where A
// is column-major k x m and B column-major k x n, both with leading dimension
// k.  Row-major [m, k] weights and row-major [n, k] tokens are exactly such
// A and B, and D then holds one token per column.
mlstm_status_t gemm_tn(int dev, int m, int n, int k, const void *A, const void *Bm, void *D,
                       hipDataType ab, hipDataType dt, const float *bias, void *ws, hipStream_t s) {
    hipblasLtHandle_t h = handle_for(dev);
    if (!h) return MLSTM_ERR_BLAS;
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
    hipblasLtMatmulPreference_t pref = nullptr;
    mlstm_status_t st = MLSTM_ERR_BLAS;
    const hipblasOperation_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
    const hipblasLtEpilogue_t epi = bias ? HIPBLASLT_EPILOGUE_BIAS : HIPBLASLT_EPILOGUE_DEFAULT;
    const hipDataType bias_t = HIP_R_32F;
    const uint64_t wsb = kGemmWorkspace;
    const float alpha = 1.0f, beta = 0.0f;
    hipblasLtMatmulAlgo_t algo{};
    bool have = false;
    do {
        if (hipblasLtMatmulDescCreate(&desc, HIPBLAS_COMPUTE_32F, HIP_R_32F)) break;
        if (hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof(opT))) break;
        if (hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opN, sizeof(opN))) break;
        if (hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi, sizeof(epi))) break;
        if (bias) {
            if (hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias, sizeof(bias)))
                break;
            if (hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &bias_t,
                                                sizeof(bias_t)))
                break;
        }
        if (hipblasLtMatrixLayoutCreate(&la, ab, k, m, k)) break;
        if (hipblasLtMatrixLayoutCreate(&lb, ab, k, n, k)) break;
        if (hipblasLtMatrixLayoutCreate(&ld, dt, m, n, m)) break;
        const AlgoKey key{dev, m, n, k, (int)ab, (int)dt, bias != nullptr};
        {
            std::lock_guard<std::mutex> lk(g_mu);
            auto it = g_algo.find(key);
            if (it != g_algo.end()) {
                algo = it->second;
                have = true;
            }
        }
        if (!have) {
            if (hipblasLtMatmulPreferenceCreate(&pref)) break;
            if (hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb,
                                                      sizeof(wsb)))
                break;
            hipblasLtMatmulHeuristicResult_t res[1];
            int found = 0;
            if (hipblasLtMatmulAlgoGetHeuristic(h, desc, la, lb, ld, ld, pref, 1, res, &found) || found < 1)
                break;
            algo = res[0].algo;
            std::lock_guard<std::mutex> lk(g_mu);
            g_algo[key] = algo;
        }
        if (hipblasLtMatmul(h, desc, &alpha, A, la, Bm, lb, &beta, D, ld, D, ld, &algo, ws, kGemmWorkspace, s))
            break;
        st = MLSTM_OK;
    } while (false);
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    if (ld) hipblasLtMatrixLayoutDestroy(ld);
    if (lb) hipblasLtMatrixLayoutDestroy(lb);
    if (la) hipblasLtMatrixLayoutDestroy(la);
    if (desc) hipblasLtMatmulDescDestroy(desc);
    return st;
}

struct LayerPlan {
    size_t es, BT, nq, nv, ng;           // element size; tokens; q/k, v/o, gate element counts
    size_t off_q, off_k, off_v, off_o, off_i, off_f, off_wg, off_cell, cell_bytes, total;
    bool all_heads;                      // one GEMM per weight over all heads (strided rows)
    bool one_gate_gemm;                  // W_i and W_f stacked: one gate GEMM
};

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

mlstm_status_t layer_plan(int B, int T, int D, int H, int dk, int dv, int chunk, mlstm_dtype_t io,
                          LayerPlan *p) {
    if (B <= 0 || T <= 0 || D <= 0 || H <= 0 || dk <= 0 || dv <= 0) return MLSTM_ERR_SHAPE;
    if (io != MLSTM_F32 && io != MLSTM_BF16) return MLSTM_ERR_UNSUPPORTED;
    if (D % 8 != 0) return MLSTM_ERR_UNSUPPORTED;  // rows of x and W 16-byte aligned
    size_t BT, HBT;
    if (!mul_ok((size_t)B, (size_t)T, &BT) || BT > (size_t)INT32_MAX) return MLSTM_ERR_SHAPE;
    if (!mul_ok(BT, (size_t)H, &HBT) || HBT > ((size_t)1 << 40)) return MLSTM_ERR_SHAPE;
    size_t cell = 0;
    mlstm_status_t st = mlstm_fwd_chunkwise_workspace_size(H, B, T, dk, dv, chunk, io, &cell);
    if (st != MLSTM_OK) return st;
    p->es = io == MLSTM_BF16 ? 2 : 4;
    p->BT = BT;
    p->nq = HBT * dk;
    p->nv = HBT * dv;
    p->ng = HBT;
    p->off_q = kGemmWorkspace;
    p->off_k = p->off_q + up256(p->nq * p->es);
    p->off_v = p->off_k + up256(p->nq * p->es);
    p->off_o = p->off_v + up256(p->nv * p->es);
    // the gate pre-activations: [H][B*T] float32 each, i~ then f~; adjacent
    // (one GEMM writes both) when f~ stays 16-byte aligned that way
    p->all_heads = ws_kernel_selected(io == MLSTM_BF16, dk, dv, prefill_kernel_chunk(io == MLSTM_BF16, dk, dv, chunk));
    p->one_gate_gemm = p->all_heads && p->ng % 4 == 0;
    p->off_i = p->off_o + up256(p->nv * p->es);
    p->off_f = p->off_i + (p->one_gate_gemm ? p->ng * 4 : up256(p->ng * 4));
    p->off_wg = p->off_i + 2 * up256(p->ng * 4);           // W_i, W_f stacked [2H, D]
    p->off_cell = p->off_wg + up256(2 * (size_t)H * D * p->es);
    p->cell_bytes = cell;
    p->total = p->off_cell + up256(cell);
    return MLSTM_OK;
}

}  // namespace
}  // namespace mlstm

using namespace mlstm;

extern "C" {

mlstm_status_t mlstm_layer_fwd_workspace_size(int B, int T, int d_model, int H, int d_qk, int d_v,
                                              int chunk, mlstm_dtype_t io, size_t *bytes) {
    if (!bytes) return MLSTM_ERR_NULL;
    *bytes = 0;
    LayerPlan p;
    const mlstm_status_t st = layer_plan(B, T, d_model, H, d_qk, d_v, chunk, io, &p);
    if (st == MLSTM_OK) *bytes = p.total;
    return st;
}

mlstm_status_t mlstm_layer_fwd(const void *x, const void *W_q, const void *W_k, const void *W_v,
                               const void *W_o, const void *W_i, const void *W_f, const float *b_q,
                               const float *b_k, const float *b_v, const float *b_o, const float *b_i,
                               const float *b_f, const float *C0, const float *n0, const float *m0,
                               void *h, float *C_T, float *n_T, float *m_T, int B, int T, int d_model,
                               int H, int d_qk, int d_v, int chunk, mlstm_dtype_t io, void *workspace,
                               size_t workspace_bytes, void *stream) {
    if (!x || !W_q || !W_k || !W_v || !W_o || !W_i || !W_f || !b_q || !b_k || !b_v || !b_o || !b_i ||
        !b_f || !h)
        return MLSTM_ERR_NULL;
    LayerPlan p;
    mlstm_status_t st = layer_plan(B, T, d_model, H, d_qk, d_v, chunk, io, &p);
    if (st != MLSTM_OK) return st;
    // Every check of the cell call at the end runs here as well, before the
    // first GEMM is enqueued: a rejected call enqueues nothing.
    const int in0 = (C0 != nullptr) + (n0 != nullptr) + (m0 != nullptr);
    const int out0 = (C_T != nullptr) + (n_T != nullptr) + (m_T != nullptr);
    if ((in0 != 0 && in0 != 3) || (out0 != 0 && out0 != 3)) return MLSTM_ERR_STATE_ARGS;
    if (!all_aligned({x, W_q, W_k, W_v, W_o, W_i, W_f, b_q, b_k, b_v, b_o, b_i, b_f, C0, n0, m0, h, C_T,
                      n_T, m_T, workspace}))
        return MLSTM_ERR_ALIGN;
    if (!workspace || workspace_bytes < p.total) return MLSTM_ERR_WORKSPACE;
    const size_t es = p.es, D = (size_t)d_model;
    const Range ins[] = {rng(x, p.BT * D * es),           rng(W_q, (size_t)H * d_qk * D * es),
                         rng(W_k, (size_t)H * d_qk * D * es), rng(W_v, (size_t)H * d_v * D * es),
                         rng(W_o, (size_t)H * d_v * D * es),  rng(W_i, (size_t)H * D * es),
                         rng(W_f, (size_t)H * D * es),        rng(b_q, (size_t)H * d_qk * 4),
                         rng(b_k, (size_t)H * d_qk * 4),      rng(b_v, (size_t)H * d_v * 4),
                         rng(b_o, (size_t)H * d_v * 4),       rng(b_i, (size_t)H * 4),
                         rng(b_f, (size_t)H * 4)};
    const size_t nC = (size_t)H * B * d_qk * d_v, nn = (size_t)H * B * d_qk, nm = (size_t)H * B;
    const Range st_in[] = {rng(C0, nC * 4), rng(n0, nn * 4), rng(m0, nm * 4)};
    // written: h, the final state and the workspace
    const Range outs[] = {rng(h, p.nv * es), rng(C_T, nC * 4), rng(n_T, nn * 4), rng(m_T, nm * 4),
                          rng(workspace, p.total)};
    constexpr int NO = sizeof(outs) / sizeof(outs[0]);
    for (const Range &o : outs) {
        for (const Range &i : ins)
            if (overlaps(i, o)) return MLSTM_ERR_ALIAS;
    }
    // each written buffer overlaps no other one; a final-state buffer may
    // coincide exactly with its own initial-state buffer (in place) and
    // overlaps no other initial-state buffer
    for (int o = 0; o < NO; ++o) {
        for (int o2 = o + 1; o2 < NO; ++o2)
            if (overlaps(outs[o], outs[o2])) return MLSTM_ERR_ALIAS;
        for (int i = 0; i < 3; ++i) {
            const bool allowed = o == i + 1 && same(outs[o], st_in[i]);
            if (overlaps(outs[o], st_in[i]) && !allowed) return MLSTM_ERR_ALIAS;
        }
    }

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MLSTM_ERR_HIP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    const hipDataType ab = io == MLSTM_BF16 ? HIP_R_16BF : HIP_R_32F;
    char *q = ws + p.off_q, *k = ws + p.off_k, *v = ws + p.off_v, *o = ws + p.off_o;
    float *gi = reinterpret_cast<float *>(ws + p.off_i), *gf = reinterpret_cast<float *>(ws + p.off_f);
    const char *Wq = static_cast<const char *>(W_q), *Wk = static_cast<const char *>(W_k);
    const char *Wv = static_cast<const char *>(W_v), *Wo = static_cast<const char *>(W_o);
    const int N = (int)p.BT;

    if (p.all_heads) {
        // one GEMM per weight: column-major [H*d, B*T], i.e. token n = b*T + t
        // holds the features of every head in one row of H*d (the cell reads
        // these strided rows directly)
        if ((st = gemm_tn(dev, H * d_qk, N, d_model, Wq, x, q, ab, ab, b_q, ws, s))) return st;
        if ((st = gemm_tn(dev, H * d_qk, N, d_model, Wk, x, k, ab, ab, b_k, ws, s))) return st;
        if ((st = gemm_tn(dev, H * d_v, N, d_model, Wv, x, v, ab, ab, b_v, ws, s))) return st;
        if ((st = gemm_tn(dev, H * d_v, N, d_model, Wo, x, o, ab, ab, b_o, ws, s))) return st;
    }
    // otherwise per head: head hh of q is the column-major [d_qk, B*T] block at hh*B*T*d_qk
    for (int hh = 0; hh < (p.all_heads ? 0 : H); ++hh) {
        const size_t wq = (size_t)hh * d_qk * D * es, wv = (size_t)hh * d_v * D * es;
        const size_t oq = (size_t)hh * p.BT * d_qk * es, ov = (size_t)hh * p.BT * d_v * es;
        if ((st = gemm_tn(dev, d_qk, N, d_model, Wq + wq, x, q + oq, ab, ab, b_q + (size_t)hh * d_qk, ws, s)))
            return st;
        if ((st = gemm_tn(dev, d_qk, N, d_model, Wk + wq, x, k + oq, ab, ab, b_k + (size_t)hh * d_qk, ws, s)))
            return st;
        if ((st = gemm_tn(dev, d_v, N, d_model, Wv + wv, x, v + ov, ab, ab, b_v + (size_t)hh * d_v, ws, s)))
            return st;
        if ((st = gemm_tn(dev, d_v, N, d_model, Wo + wv, x, o + ov, ab, ab, b_o + (size_t)hh * d_v, ws, s)))
            return st;
    }
    // gate pre-activations: [B*T, H] column-major = [H][B*T], float32; with
    // W_i and W_f stacked, one GEMM [B*T, 2H] writes i~ and then f~ (x read once)
    if (p.one_gate_gemm) {
        char *wg = ws + p.off_wg;
        const size_t wb = (size_t)H * D * es;
        if (hipMemcpyAsync(wg, W_i, wb, hipMemcpyDeviceToDevice, s) != hipSuccess ||
            hipMemcpyAsync(wg + wb, W_f, wb, hipMemcpyDeviceToDevice, s) != hipSuccess)
            return MLSTM_ERR_HIP;
        if ((st = gemm_tn(dev, N, 2 * H, d_model, x, wg, gi, ab, HIP_R_32F, nullptr, ws, s))) return st;
    } else {
        if ((st = gemm_tn(dev, N, H, d_model, x, W_i, gi, ab, HIP_R_32F, nullptr, ws, s))) return st;
        if ((st = gemm_tn(dev, N, H, d_model, x, W_f, gf, ab, HIP_R_32F, nullptr, ws, s))) return st;
    }
    hipLaunchKernelGGL(gate_bias_kernel, dim3(1024), dim3(256), 0, s, gi, gf, b_i, b_f, p.BT, H);
    if (hipGetLastError() != hipSuccess) return MLSTM_ERR_HIP;

    // the cell over the H*B head-major cells: its "B" is H and its "H" is B;
    // with all-heads projections, cell p = h*B + b reads the head-h part of
    // rows b*T .. b*T + T - 1
    if (p.all_heads) {
        const RowLayout lq{d_qk, (long long)T * H * d_qk, H * d_qk, B};
        const RowLayout lv{d_v, (long long)T * H * d_v, H * d_v, B};
        return fwd_chunkwise_rows(q, k, v, gi, gf, o, C0, n0, m0, h, C_T, n_T, m_T, H, B, T, d_qk, d_v,
                                  chunk, io, MLSTM_VARIANT_AUTO, ws + p.off_cell, p.cell_bytes, stream,
                                  &lq, &lv);
    }
    return mlstm_fwd_chunkwise(q, k, v, gi, gf, o, C0, n0, m0, h, C_T, n_T, m_T, H, B, T, d_qk, d_v,
                               chunk, io, ws + p.off_cell, p.cell_bytes, stream);
}

}  // extern "C"
