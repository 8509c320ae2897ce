// step.hip -- one recurrent step of the mLSTM cell (decode), gfx950.
//
// Per (batch, head) pair, with the state in stabilized variables (xLSTM note,
// "sLSTM" section for the stabilizer, "mLSTM (matrix LSTM)" section for the
// memory, normalizer and read-out):
//   m'  = max(f~ + m, i~),  f' = e^{f~ + m - m'},  i' = e^{i~ - m'}
//   C'  = f' C' + i' k v^T          (d_qk x d_v, float32, updated in place)
//   n'  = f' n' + i' k
//   h   = sigmoid(o~) * (C'^T q) / max(|n'^T q|, e^{-m'})
//
// The step is bound by HBM: each pair streams its d_qk*d_v float32 memory
// once in and once out (512 KiB each way per pair at 256x512), against ~5 flops per
// element.  One workgroup owns one pair, so the in-place update of n and m
// cannot race with another workgroup.  Threads are laid out as TPR = d_v/4
// column groups (one float4 of a row each) times RPI = NTH/TPR row groups, so
// a wavefront reads 64 consecutive float4 of one row (1 KiB, fully
// coalesced); each thread keeps UNROLL rows of loads in flight, and the
// read-out C'^T q is accumulated in the same pass and reduced over row groups
// through LDS.
#include "common.hpp"

namespace mlstm {

namespace {

constexpr int NTH = 512;
constexpr int UNROLL = 8;

// streaming (non-temporal) 16-byte accesses: the memory is touched once per step
__device__ __forceinline__ f32x4 ld_c(const float *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
}
__device__ __forceinline__ void st_c(float *p, f32x4 x) {
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(p));
}

template <typename IO>
__global__ __launch_bounds__(NTH) void mlstm_step_kernel(StepArgs a) {
    const int bh = blockIdx.x;
    const int tid = threadIdx.x;
    const int dk = a.dk, dv = a.dv;
    const int TPR = dv >> 2;        // threads per row (one float4 each)
    const int RPI = NTH / TPR;      // rows per iteration
    const int c4 = tid % TPR;       // my float4 column
    const int r0 = tid / TPR;       // my first row

    __shared__ float qs[256], ks[256];
    __shared__ __attribute__((aligned(16))) float red[NTH * 4];  // RPI x d_v partial read-outs (= 1024 floats)
    __shared__ float nq_part[NTH / 64];

    const IO *q = static_cast<const IO *>(a.q) + (size_t)bh * dk;
    const IO *k = static_cast<const IO *>(a.k) + (size_t)bh * dk;
    const IO *v = static_cast<const IO *>(a.v) + (size_t)bh * dv;
    const IO *o = static_cast<const IO *>(a.o) + (size_t)bh * dv;
    for (int i = tid; i < dk; i += NTH) {
        qs[i] = to_f(q[i]);
        ks[i] = to_f(k[i]);
    }
    const float m_old = a.m_in ? a.m_in[bh] : 0.0f;
    const float ig = a.ig[bh], fg = a.fg[bh];
    const float m_new = fmaxf(fg + m_old, ig);
    const float fp = exp_e(fg + m_old - m_new);
    const float ip = exp_e(ig - m_new);

    // when TPR does not divide the block, the last few threads own no column
    const bool active = r0 < RPI;
    f32x4 vv = {0.f, 0.f, 0.f, 0.f};
    if (active)
        vv = f32x4{to_f(v[4 * c4 + 0]), to_f(v[4 * c4 + 1]), to_f(v[4 * c4 + 2]), to_f(v[4 * c4 + 3])};
    __syncthreads();

    const size_t base = (size_t)bh * dk * dv + 4 * c4;
    const float *Cin = a.C_in ? a.C_in + base : nullptr;
    float *Cout = a.C_out + base;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};

    // rows r0, r0 + RPI, ...; UNROLL of them per batch so their loads overlap
    for (int a0 = active ? r0 : dk; a0 < dk; a0 += RPI * UNROLL) {
        f32x4 cv[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int row = a0 + u * RPI;
            cv[u] = (Cin && row < dk) ? ld_c(Cin + (size_t)row * dv) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int row = a0 + u * RPI;
            if (row < dk) {
                const float ik = ip * ks[row];
                const float qa = qs[row];
                f32x4 c = cv[u];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    c[e] = fmaf(fp, c[e], ik * vv[e]);
                    acc[e] = fmaf(c[e], qa, acc[e]);
                }
                st_c(Cout + (size_t)row * dv, c);
            }
        }
    }
    if (active) *reinterpret_cast<f32x4 *>(&red[r0 * dv + 4 * c4]) = acc;

    // normalizer: thread a owns n[a] (read and written by the same thread)
    float nq = 0.0f;
    for (int i = tid; i < dk; i += NTH) {
        const float n_old = a.n_in ? a.n_in[(size_t)bh * dk + i] : 0.0f;
        const float n_new = fmaf(fp, n_old, ip * ks[i]);
        a.n_out[(size_t)bh * dk + i] = n_new;
        nq = fmaf(n_new, qs[i], nq);
    }
    for (int off = 32; off > 0; off >>= 1) nq += __shfl_xor(nq, off, 64);
    if ((tid & 63) == 0) nq_part[tid >> 6] = nq;
    __syncthreads();

    float nq_all = 0.0f;
#pragma unroll
    for (int w = 0; w < NTH / 64; ++w) nq_all += nq_part[w];
    const float inv = 1.0f / fmaxf(fabsf(nq_all), exp_e(-m_new));

    IO *h = static_cast<IO *>(a.h) + (size_t)bh * dv;
    for (int b = tid; b < dv; b += NTH) {
        float num = 0.0f;
        for (int r = 0; r < RPI; ++r) num += red[r * dv + b];
        h[b] = from_f<IO>(sigmoid(to_f(o[b])) * num * inv);
    }
    // every thread read m_in before the barrier above: safe to overwrite in place
    if (tid == 0) a.m_out[bh] = m_new;
}

}  // namespace

hipError_t launch_step(const StepArgs &a, int io_bf16, hipStream_t s) {
    dim3 grid(a.BH), block(NTH);
    if (io_bf16)
        hipLaunchKernelGGL(mlstm_step_kernel<bf16>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(mlstm_step_kernel<float>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace mlstm
