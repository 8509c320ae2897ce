// backward.hip -- reverse mode of the mLSTM cell (gradients of a loss whose
// gradient with respect to h is given), gfx950.
//
// Mathematics (xLSTM note, "mLSTM (matrix LSTM)" and "sLSTM" sections, the
// same recurrence as the forward): in the unstabilized variables the
// read-out is C q / max(|n^T q|, 1), so the stabilizer m is not
// differentiated and the gradients are carried in the stabilized variables.
// Per token, with den_t the forward's denominator,
//   a_t    = dh_t * sigmoid(o~_t) / den_t
//   beta_t = -sign(n_t.q_t) (a_t . num_t) / den_t   (0 when the floor is active)
//   dq_t   = C_t a_t + n_t beta_t
//   dk_t   = i'_t (dC*_t v_t + dn*_t),   dv_t = i'_t dC*_t^T k_t
//   do~_t  = dh_t * num_t / den_t * sigmoid'(o~_t)
//   di~_t  = k_t . dk_t,   df~_t = sum_{s >= t} (q_s . dq_s - k_s . dk_s)
// where dC*_t = q_t a_t^T + f'_{t+1} dC*_{t+1} (and dn*_t likewise with
// beta) runs backwards in time with the forward's own decay factors.
//
// Chunkwise, per chunk of L tokens with the forward's in-chunk quantities
// (b = cumsum f~, u_j = i~_j - b_j, r_i = max(m_prev, max_{j<=i} u_j), so
// m_t = b_i + r_i) and the carried gradient G* (stabilized at the chunk's
// last token, m_c = b_{L-1} + r_{L-1}):
//   P_ij  = (q_i.k_j) e^{u_j - r_i},   P~_ij = (a_i.v_j + beta_i) e^{u_j - r_i}   (j <= i)
//   num_i = e^{m_prev - r_i} C'^T q_i + sum_j P_ij v_j     (C', n': state at the chunk start)
//   dq_i  = e^{m_prev - r_i} (C' a_i + n' beta_i) + sum_j P~_ij k_j
//   dk_j  = sum_i P~_ij q_i + w_j (G* v_j + g*),   dv_j = sum_i P_ij a_i + w_j G*^T k_j
//   G*   <- e^{m_prev - r_{L-1}} G* + sum_i e^{m_prev - r_i} q_i a_i^T   (g* likewise)
// with w_j = e^{u_j - r_{L-1}}; after the first chunk G* and g* are the
// gradients of the initial state (C0, n0) and dm0 = <dC0, C0> + dn0 . n0.
//
// Two launches.  The first runs the forward state recurrence per pair and
// stores the state (C', n', m) at every chunk start in the workspace; the
// second walks the chunks backwards.  One workgroup owns one pair and keeps
// its tiles, the chunk-start state and G* in LDS (float32 throughout), so
// this version covers d_qk, d_v <= 64.
#include "common.hpp"

namespace mlstm {

namespace {

constexpr int L = kBwdChunk, D = kBwdMaxDim, NTH = 256;

// In-chunk gate quantities of tokens t0 .. t0 + L - 1 for the stabilizer
// m_before, by one wavefront (lane j = token j; tokens past T act as i~ =
// -inf, f~ = 0, which leaves every running quantity unchanged):
// gb = cumsum f~, gu = i~ - gb, gr = max(m_before, prefix max gu); last =
// (gb, gr) of the chunk's last token.
__device__ void chunk_gates(const float *ig, const float *fg, int t0, int T, float m_before, float *gb,
                            float *gu, float *gr, float *last) {
    const int lane = threadIdx.x & 63;
    const int t = t0 + lane;
    const bool ok = lane < L && t < T;
    float b = ok ? fg[t] : 0.0f;
    const float i = ok ? ig[t] : -INFINITY;
    for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(b, o, 64);
        if (lane >= o) b += y;
    }
    const float u = i - b;
    float pm = u;
    for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(pm, o, 64);
        if (lane >= o) pm = fmaxf(pm, y);
    }
    const float r = fmaxf(m_before, pm);
    if (lane < L) {
        gb[lane] = b;
        gu[lane] = u;
        gr[lane] = r;
    }
    if (lane == L - 1) {
        last[0] = b;
        last[1] = r;
    }
}

template <typename IO>
__global__ __launch_bounds__(NTH) void bwd_ckpt_kernel(BwdArgs a) {
    __shared__ float Cs[D * D], ns[D], Kt[L * D], Vt[L * D], wv[L], gb[L], gu[L], gr[L], last[2];
    const int p = blockIdx.x, tid = threadIdx.x;
    const int dk = a.dk, dv = a.dv, T = a.T;
    const int nch = (T + L - 1) / L;
    const size_t rec = (size_t)dk * dv + dk + 1;
    const IO *kg = static_cast<const IO *>(a.k) + (size_t)p * T * dk;
    const IO *vg = static_cast<const IO *>(a.v) + (size_t)p * T * dv;
    const float *igp = a.ig + (size_t)p * T, *fgp = a.fg + (size_t)p * T;

    for (int e = tid; e < dk * dv; e += NTH) Cs[e] = a.C0 ? a.C0[(size_t)p * dk * dv + e] : 0.0f;
    for (int e = tid; e < dk; e += NTH) ns[e] = a.n0 ? a.n0[(size_t)p * dk + e] : 0.0f;
    float m = a.m0 ? a.m0[p] : 0.0f;
    __syncthreads();
    float *ck = a.ckpt + (size_t)p * nch * rec;
    for (int c = 0; c < nch; ++c) {
        const int t0 = c * L;
        float *r = ck + (size_t)c * rec;
        for (int e = tid; e < dk * dv; e += NTH) r[e] = Cs[e];
        for (int e = tid; e < dk; e += NTH) r[(size_t)dk * dv + e] = ns[e];
        if (tid == 0) r[(size_t)dk * dv + dk] = m;
        for (int e = tid; e < L * dk; e += NTH) {
            const int t = t0 + e / dk;
            Kt[e] = t < T ? to_f(kg[(size_t)t * dk + e % dk]) : 0.0f;
        }
        for (int e = tid; e < L * dv; e += NTH) {
            const int t = t0 + e / dv;
            Vt[e] = t < T ? to_f(vg[(size_t)t * dv + e % dv]) : 0.0f;
        }
        if (tid < 64) chunk_gates(igp, fgp, t0, T, m, gb, gu, gr, last);
        __syncthreads();
        const float b_last = last[0], r_last = last[1];
        const float dec = exp_e(m - r_last);
        if (tid < L) wv[tid] = exp_e(gu[tid] - r_last);
        __syncthreads();
        for (int e = tid; e < dk * dv; e += NTH) {
            const int row = e / dv, col = e % dv;
            float acc = dec * Cs[e];
            for (int j = 0; j < L; ++j) acc = fmaf(wv[j] * Kt[j * dk + row], Vt[j * dv + col], acc);
            Cs[e] = acc;
        }
        for (int e = tid; e < dk; e += NTH) {
            float acc = dec * ns[e];
            for (int j = 0; j < L; ++j) acc = fmaf(wv[j], Kt[j * dk + e], acc);
            ns[e] = acc;
        }
        m = b_last + r_last;
        __syncthreads();
    }
}

template <typename IO>
__global__ __launch_bounds__(NTH) void bwd_kernel(BwdArgs a) {
    __shared__ float Q[L * D], K[L * D], V[L * D], SG[L * D], DH[L * D], NUM[L * D], A[L * D], DQ[L * D],
        DK[L * D];
    __shared__ float Cc[D * D], Gs[D * D], P[L * L], PT[L * L];
    __shared__ float nc[D], gs[D], gb[L], gu[L], gr[L], sv[L], fl[L], wv[L], dd[L], den[L], beta[L];
    __shared__ float last[2], carry, red[NTH];
    const int p = blockIdx.x, tid = threadIdx.x;
    const int dk = a.dk, dv = a.dv, T = a.T;
    const int nch = (T + L - 1) / L;
    const size_t rec = (size_t)dk * dv + dk + 1;
    const size_t oqk = (size_t)p * T * dk, ov = (size_t)p * T * dv, og1 = (size_t)p * T;
    const IO *qg = static_cast<const IO *>(a.q) + oqk;
    const IO *kg = static_cast<const IO *>(a.k) + oqk;
    const IO *vg = static_cast<const IO *>(a.v) + ov;
    const IO *ogp = static_cast<const IO *>(a.o) + ov;
    const IO *dhg = static_cast<const IO *>(a.dh) + ov;

    for (int e = tid; e < dk * dv; e += NTH) Gs[e] = 0.0f;
    for (int e = tid; e < dk; e += NTH) gs[e] = 0.0f;
    if (tid == 0) carry = 0.0f;
    __syncthreads();
    for (int c = nch - 1; c >= 0; --c) {
        const int t0 = c * L;
        const float *ck = a.ckpt + ((size_t)p * nch + c) * rec;
        for (int e = tid; e < dk * dv; e += NTH) Cc[e] = ck[e];
        for (int e = tid; e < dk; e += NTH) nc[e] = ck[(size_t)dk * dv + e];
        const float m_prev = ck[(size_t)dk * dv + dk];
        for (int e = tid; e < L * dk; e += NTH) {
            const int t = t0 + e / dk;
            const size_t g = (size_t)t * dk + e % dk;
            Q[e] = t < T ? to_f(qg[g]) : 0.0f;
            K[e] = t < T ? to_f(kg[g]) : 0.0f;
        }
        for (int e = tid; e < L * dv; e += NTH) {
            const int t = t0 + e / dv;
            const size_t g = (size_t)t * dv + e % dv;
            V[e] = t < T ? to_f(vg[g]) : 0.0f;
            SG[e] = t < T ? sigmoid(to_f(ogp[g])) : 0.0f;
            DH[e] = t < T ? to_f(dhg[g]) : 0.0f;
        }
        if (tid < 64) chunk_gates(a.ig + og1, a.fg + og1, t0, T, m_prev, gb, gu, gr, last);
        __syncthreads();
        const float r_last = last[1];
        const float dec = exp_e(m_prev - r_last);
        if (tid < L) {
            sv[tid] = exp_e(m_prev - gr[tid]);
            fl[tid] = exp_e(-(gb[tid] + gr[tid]));
            wv[tid] = exp_e(gu[tid] - r_last);
        }
        // P_ij = (q_i.k_j) e^{u_j - r_i}, causal, rows of real tokens only
        for (int e = tid; e < L * L; e += NTH) {
            const int i = e / L, j = e % L;
            float s = 0.0f;
            if (j <= i && t0 + i < T) {
                for (int r = 0; r < dk; ++r) s = fmaf(Q[i * dk + r], K[j * dk + r], s);
                s *= exp_e(gu[j] - gr[i]);
            }
            P[e] = s;
        }
        __syncthreads();
        // forward read-out and denominator, recomputed
        for (int e = tid; e < L * dv; e += NTH) {
            const int i = e / dv, b = e % dv;
            float acc = 0.0f;
            for (int r = 0; r < dk; ++r) acc = fmaf(Cc[r * dv + b], Q[i * dk + r], acc);
            acc *= sv[i];
            for (int j = 0; j <= i; ++j) acc = fmaf(P[i * L + j], V[j * dv + b], acc);
            NUM[e] = acc;
        }
        if (tid < L) {
            const int i = tid;
            float acc = 0.0f;
            for (int r = 0; r < dk; ++r) acc = fmaf(nc[r], Q[i * dk + r], acc);
            acc *= sv[i];
            for (int j = 0; j <= i; ++j) acc += P[i * L + j];
            dd[i] = acc;
            den[i] = fmaxf(fabsf(acc), fl[i]);
        }
        __syncthreads();
        // a = dh sigmoid(o~) / den, and the output-gate gradient
        for (int e = tid; e < L * dv; e += NTH) {
            const int i = e / dv;
            const float sg = SG[e];
            A[e] = DH[e] * sg / den[i];
            const int t = t0 + i;
            if (t < T) a.go[ov + (size_t)t * dv + e % dv] = DH[e] * NUM[e] / den[i] * sg * (1.0f - sg);
        }
        __syncthreads();
        if (tid < L) {
            const int i = tid;
            float an = 0.0f;
            for (int b = 0; b < dv; ++b) an = fmaf(A[i * dv + b], NUM[i * dv + b], an);
            beta[i] = fabsf(dd[i]) > fl[i] ? (dd[i] > 0.0f ? -an : an) / den[i] : 0.0f;
        }
        __syncthreads();
        // P~_ij = (a_i.v_j + beta_i) e^{u_j - r_i}
        for (int e = tid; e < L * L; e += NTH) {
            const int i = e / L, j = e % L;
            float s = 0.0f;
            if (j <= i && t0 + i < T) {
                for (int b = 0; b < dv; ++b) s = fmaf(A[i * dv + b], V[j * dv + b], s);
                s = (s + beta[i]) * exp_e(gu[j] - gr[i]);
            }
            PT[e] = s;
        }
        __syncthreads();
        for (int e = tid; e < L * dk; e += NTH) {
            const int i = e / dk, r = e % dk;
            float acc = 0.0f;
            for (int b = 0; b < dv; ++b) acc = fmaf(Cc[r * dv + b], A[i * dv + b], acc);
            acc = sv[i] * fmaf(nc[r], beta[i], acc);
            for (int j = 0; j <= i; ++j) acc = fmaf(PT[i * L + j], K[j * dk + r], acc);
            DQ[e] = acc;
            const int t = t0 + i;
            if (t < T) a.gq[oqk + (size_t)t * dk + r] = acc;
        }
        for (int e = tid; e < L * dk; e += NTH) {
            const int j = e / dk, r = e % dk;
            float acc = 0.0f;
            for (int i = j; i < L; ++i) acc = fmaf(PT[i * L + j], Q[i * dk + r], acc);
            float gv = gs[r];
            for (int b = 0; b < dv; ++b) gv = fmaf(Gs[r * dv + b], V[j * dv + b], gv);
            acc = fmaf(wv[j], gv, acc);
            DK[e] = acc;
            const int t = t0 + j;
            if (t < T) a.gk[oqk + (size_t)t * dk + r] = acc;
        }
        for (int e = tid; e < L * dv; e += NTH) {
            const int j = e / dv, b = e % dv;
            float acc = 0.0f;
            for (int i = j; i < L; ++i) acc = fmaf(P[i * L + j], A[i * dv + b], acc);
            float gk = 0.0f;
            for (int r = 0; r < dk; ++r) gk = fmaf(Gs[r * dv + b], K[j * dk + r], gk);
            acc = fmaf(wv[j], gk, acc);
            const int t = t0 + j;
            if (t < T) a.gv[ov + (size_t)t * dv + b] = acc;
        }
        __syncthreads();
        // gate gradients: di = k.dk; df = reverse cumsum of q.dq - k.dk
        if (tid < 64) {
            const int j = tid, t = t0 + j;
            const bool ok = j < L && t < T;
            float di = 0.0f, x = 0.0f;
            if (ok) {
                float qd = 0.0f;
                for (int r = 0; r < dk; ++r) {
                    di = fmaf(K[j * dk + r], DK[j * dk + r], di);
                    qd = fmaf(Q[j * dk + r], DQ[j * dk + r], qd);
                }
                x = qd - di;
            }
            float y = x;  // sum over lanes >= j
            for (int o = 1; o < 64; o <<= 1) {
                const float z = __shfl_down(y, o, 64);
                if (j + o < 64) y += z;
            }
            const float cin = carry;
            if (ok) {
                a.gi[og1 + t] = di;
                a.gf[og1 + t] = y + cin;
            }
            const float tot = __shfl(y, 0, 64);
            if (j == 0) carry = cin + tot;
        }
        // carried gradients for the chunk before (every read of G*, g* is past
        // the barrier above)
        for (int e = tid; e < dk * dv; e += NTH) {
            const int r = e / dv, b = e % dv;
            float acc = dec * Gs[e];
            for (int i = 0; i < L; ++i) acc = fmaf(sv[i] * Q[i * dk + r], A[i * dv + b], acc);
            Gs[e] = acc;
        }
        for (int e = tid; e < dk; e += NTH) {
            float acc = dec * gs[e];
            for (int i = 0; i < L; ++i) acc = fmaf(sv[i] * beta[i], Q[i * dk + e], acc);
            gs[e] = acc;
        }
        __syncthreads();
    }
    // gradients of the initial state
    float part = 0.0f;
    for (int e = tid; e < dk * dv; e += NTH) {
        if (a.gC0) a.gC0[(size_t)p * dk * dv + e] = Gs[e];
        if (a.C0) part = fmaf(Gs[e], a.C0[(size_t)p * dk * dv + e], part);
    }
    for (int e = tid; e < dk; e += NTH) {
        if (a.gn0) a.gn0[(size_t)p * dk + e] = gs[e];
        if (a.n0) part = fmaf(gs[e], a.n0[(size_t)p * dk + e], part);
    }
    red[tid] = part;
    __syncthreads();
    for (int w = NTH / 2; w > 0; w >>= 1) {
        if (tid < w) red[tid] += red[tid + w];
        __syncthreads();
    }
    if (tid == 0 && a.gm0) a.gm0[p] = red[0];
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, int io_bf16, hipStream_t s) {
    dim3 grid(a.BH), block(NTH);
    if (io_bf16) {
        hipLaunchKernelGGL(bwd_ckpt_kernel<bf16>, grid, block, 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(bwd_kernel<bf16>, grid, block, 0, s, a);
    } else {
        hipLaunchKernelGGL(bwd_ckpt_kernel<float>, grid, block, 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(bwd_kernel<float>, grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace mlstm
