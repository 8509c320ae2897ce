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
// once in and once out (512 KiB each way per pair at 256x512), against ~5
// flops per element.  Threads are laid out as TPR = d_v/4 column groups (one
// float4 of a row each) times RPI = NTH/TPR row groups, so a wavefront reads
// 64 consecutive float4 of one row (1 KiB, fully coalesced); each thread keeps
// UNROLL rows of loads in flight, and the read-out C'^T q is accumulated in
// the same pass and reduced over row groups through LDS.
//
// Two launch shapes:
//  - one workgroup per pair (no workspace): the workgroup owns the pair's
//    whole memory, so n and m are updated in place without any race;
//  - row split (with a workspace): the pair's rows are cut into blocks of
//    RPI*UNROLL rows (128 KiB at 256 x 512: short, independent streams run
//    faster here than 512 KiB ones), which a fixed grid of workgroups walks,
//    each thread keeping its UNROLL row loads in flight from one block into
//    the next.  Each block updates its own rows of C' and n' and writes its partial
//    read-out (a d_v vector and its part of n'^T q) to the workspace; a second,
//    small launch sums the partials in block order and writes h and m'.  The
//    kernel boundary orders the two, so no block waits on another and m is
//    overwritten only after every block has read it.  (Handing the sum to the
//    last block through an atomic counter needs a device-scope release per
//    block, which writes back the whole L2 on this chip: 15x slower.)
#include <mutex>

#include "common.hpp"

namespace mlstm {

namespace {

constexpr int NTH = 512;
constexpr int UNROLL = 16;
// Workgroups of the row split's first launch: two per compute unit of an
// MI355X, run one after the other.  The kernel's registers (about 156 per
// thread) leave room for one 512-thread workgroup per compute unit and half
// of another, so the second starts in the free wave slots while the first's
// last wavefronts drain.  Measured at 256 x 512, 2048 pairs, 8192 blocks:
// 372.8 us per step, against 377.4 us for a workgroup per block, 392 us with
// 384 workgroups (uneven shares) and 377.6 us with 768.
constexpr int kStepGrid = 512;

// buffer descriptor word 3 (32-bit data format) and the non-temporal cache
// policy of the row-split kernel's buffer accesses
constexpr int kBufFlags = 0x00020000;
constexpr int kNT = 2;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// streaming (non-temporal) 16-byte accesses: the memory is touched once per step
__device__ __forceinline__ f32x4 ld_c(const float *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
}
__device__ __forceinline__ void st_c(float *p, f32x4 x) {
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(p));
}

// four consecutive I/O values (8 or 16 bytes, aligned) as float32 and back
__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ f32x4 ld4(const bf16 *p) {
    const bf16x4 x = *reinterpret_cast<const bf16x4 *>(p);
    return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}
__device__ __forceinline__ void st4(float *p, f32x4 y) { *reinterpret_cast<f32x4 *>(p) = y; }
__device__ __forceinline__ void st4(bf16 *p, f32x4 y) {
    *reinterpret_cast<bf16x4 *>(p) = bf16x4{(bf16)y[0], (bf16)y[1], (bf16)y[2], (bf16)y[3]};
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
    if (active) vv = ld4(v + 4 * c4);
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
                const f32x4 c = fp * cv[u] + (ip * ks[row]) * vv;
                acc += c * qs[row];
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

// Row split, first launch.  Block (pair, blk) covers rows [lo, lo + nr) of
// the pair's memory, at most RPI*UNROLL of them, so each thread owns at most
// UNROLL rows of it.  The grid is kStepGrid workgroups (fewer for small
// batches); workgroup g takes blocks g, g + grid, g + 2 grid, ... in turn
// and keeps every thread's UNROLL row loads in flight across them: each row
// slot is reloaded with the next block's row as soon as this block's value in
// it has been used.  The loads of the next block then overlap this block's
// stores, read-out reduction and partial write, which a workgroup per block
// pays for with idle memory slots at its start and end.  Each block writes
// its rows of C' and n' and its partial read-out (d_v values, then its part
// of n'^T q).  Every block's arithmetic and the order of its sums are those
// of a workgroup per block.
template <typename IO, bool STATE>
__global__ __launch_bounds__(NTH) void mlstm_step_rows_kernel(StepArgs a) {
    const int nb = a.nb;
    const int nblk = a.BH * nb;
    const int grid = gridDim.x;
    const int tid = threadIdx.x;
    const int dk = a.dk, dv = a.dv;
    const int TPR = dv >> 2, RPI = NTH / TPR;
    const int c4 = tid % TPR, r0 = tid / TPR;
    const bool active = r0 < RPI;
    const int rstep = RPI * dv * 4;

    __shared__ float qs[256], ks[256];
    __shared__ __attribute__((aligned(16))) float red[NTH * 4];
    __shared__ float nq_part[2][NTH / 64];  // by block parity: thread 0 may still read the last one

    // a block's rows, and its small loads: the thread's q, k, n rows (at an
    // index clamped into the block: the surplus is never used), the pair's v
    // group and gate scalars
    struct Rows {
        int bh, blk, nr;
        size_t pk;
    };
    auto rows_of = [&](int i) {
        Rows r;
        r.bh = i / nb;
        r.blk = i - r.bh * nb;
        const int lo = r.blk * a.rows;
        r.nr = min(dk - lo, a.rows);
        r.pk = (size_t)r.bh * dk + lo;
        return r;
    };
    struct Small {
        IO qr, kr;
        float nv, m_old, ig, fg;
        f32x4 vv;
    };
    auto small = [&](const Rows &r) {
        const int tr = min(tid, r.nr - 1);
        Small x;
        x.qr = static_cast<const IO *>(a.q)[r.pk + tr];
        x.kr = static_cast<const IO *>(a.k)[r.pk + tr];
        x.nv = STATE ? a.n_in[r.pk + tr] : 0.0f;
        x.vv = ld4(static_cast<const IO *>(a.v) + (size_t)r.bh * dv + 4 * c4);
        x.m_old = STATE ? a.m_in[r.bh] : 0.0f;
        x.ig = a.ig[r.bh];
        x.fg = a.fg[r.bh];
        return x;
    };
    // A block's rows of C' through buffer descriptors: one 32-bit lane offset
    // per row instead of a 64-bit address (registers for the loads in
    // flight), and the hardware's range check on the block turns rows past
    // its end (and idle lanes, aimed past it) into zero loads and dropped
    // stores.  An empty range reads nothing at all.
    const float *cin = STATE ? a.C_in : a.C_out;  // (not read without a state)
    auto c_rsrc = [&](float *base, const Rows &r, int nbytes) {
        return __builtin_amdgcn_make_buffer_rsrc(base + r.pk * dv, 0, __builtin_amdgcn_readfirstlane(nbytes), kBufFlags);
    };
    auto lane_off = [&](const Rows &r) { return active ? (r0 * dv + 4 * c4) * 4 : r.nr * dv * 4; };

    int i = blockIdx.x;
    Rows cur = rows_of(i);
    Small sc = small(cur);
    f32x4 cv[UNROLL];
    {
        const auto rin = c_rsrc(const_cast<float *>(cin), cur, cur.nr * dv * 4);
        const int voff = lane_off(cur);
        __builtin_amdgcn_sched_barrier(0);  // keep the issue order: small loads, then the memory's
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            if constexpr (STATE)
                cv[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rin, voff + u * rstep, 0, kNT));
            else
                cv[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int par = 0;; par ^= 1) {
        const int inext = i + grid;
        const bool more = inext < nblk;
        const float m_new = fmaxf(sc.fg + sc.m_old, sc.ig);
        const float fp = exp_e(sc.fg + sc.m_old - m_new);
        const float ip = exp_e(sc.ig - m_new);

        // normalizer rows (thread r owns row lo + r) and q, k rows for the update
        float nq = 0.0f;
        if (tid < cur.nr) {
            const float qv = to_f(sc.qr), kv = to_f(sc.kr);
            qs[tid] = qv;
            ks[tid] = kv;
            const float n_new = fmaf(fp, sc.nv, ip * kv);
            a.n_out[cur.pk + tid] = n_new;
            nq = n_new * qv;
        }
        for (int off = 32; off > 0; off >>= 1) nq += __shfl_xor(nq, off, 64);
        if ((tid & 63) == 0) nq_part[par][tid >> 6] = nq;
        __syncthreads();

        // The next block's small loads and row loads are issued whether or
        // not there is a next block: past the last one they reload this
        // block's small values and read an empty range (a conditional load
        // would keep the old and the new value of each slot alive together).
        const Rows nxt = rows_of(more ? inext : i);
        const Small sn = small(nxt);
        const auto rnext = c_rsrc(const_cast<float *>(cin), nxt, more ? nxt.nr * dv * 4 : 0);
        const int noff = lane_off(nxt);
        const auto rout = c_rsrc(a.C_out, cur, cur.nr * dv * 4);
        const int voff = lane_off(cur);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int r = r0 + u * RPI;
            if (active && r < cur.nr) {
                const f32x4 c = fp * cv[u] + (ip * ks[r]) * sc.vv;
                acc += c * qs[r];
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, c), rout, voff + u * rstep, 0, kNT);
            }
            if constexpr (STATE)
                cv[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rnext, noff + u * rstep, 0, kNT));
            __builtin_amdgcn_sched_barrier(0);  // slot u is reloaded only after its use
        }
        if (active) *reinterpret_cast<f32x4 *>(&red[r0 * dv + 4 * c4]) = acc;
        __syncthreads();

        float *pp = a.part + ((size_t)cur.bh * nb + cur.blk) * (dv + 4);
        for (int b = tid; b < dv; b += NTH) {
            float num = 0.0f;
            for (int r = 0; r < RPI; ++r) num += red[r * dv + b];
            pp[b] = num;
        }
        if (tid == 0) {
            float nq_all = 0.0f;
#pragma unroll
            for (int w = 0; w < NTH / 64; ++w) nq_all += nq_part[par][w];
            pp[dv] = nq_all;
        }
        if (!more) break;
        // (qs, ks and red are rewritten only after the next block's first
        // barrier, which every thread reaches after its reads of them here)
        i = inext;
        cur = nxt;
        sc = sn;
    }
}

// Row split, second launch: per pair, the partials summed in block order, the
// gated read-out h and the new stabilizer (written here, after every block of
// the pair has read the old one).  One thread per float4 of h.
template <typename IO>
__global__ __launch_bounds__(128) void mlstm_step_finish_kernel(StepArgs a) {
    const int bh = blockIdx.x;
    const int nb = a.nb, dv = a.dv, ld = dv + 4;
    const float *pp = a.part + (size_t)bh * nb * ld;
    const float m_old = a.m_in ? a.m_in[bh] : 0.0f;
    const float m_new = fmaxf(a.fg[bh] + m_old, a.ig[bh]);
    float nq = 0.0f;
    for (int j = 0; j < nb; ++j) nq += pp[j * ld + dv];
    const float inv = 1.0f / fmaxf(fabsf(nq), exp_e(-m_new));
    const IO *o = static_cast<const IO *>(a.o) + (size_t)bh * dv;
    IO *h = static_cast<IO *>(a.h) + (size_t)bh * dv;
    for (int c = threadIdx.x; c < (dv >> 2); c += blockDim.x) {
        f32x4 num = {0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < nb; ++j) num += *reinterpret_cast<const f32x4 *>(pp + j * ld + 4 * c);
        const f32x4 og = ld4(o + 4 * c);
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = sigmoid(og[e]) * num[e] * inv;
        st4(h + 4 * c, y);
    }
    // every thread read m_in above: safe to overwrite in place after the barrier
    __syncthreads();
    if (threadIdx.x == 0) a.m_out[bh] = m_new;
}

}  // namespace

int step_rows_per_block(int, int dv) {
    const int tpr = dv / 4;
    return (NTH / tpr) * UNROLL;
}

size_t step_workspace_bytes(size_t BH, int dk, int dv) {
    const int rows = step_rows_per_block(dk, dv);
    const size_t nb = ((size_t)dk + rows - 1) / rows;
    return nb < 2 ? 0 : BH * nb * (size_t)(dv + 4) * 4;
}

// Fixed scratch of the entry point that allocates nothing: the row split's
// partial read-outs, in a file-scope array of the library's code object (each
// device holds its own copy, at its own address, until the process ends).
// Host code never passes the array's name to a kernel (on the host it is only
// a stand-in for the symbol): it looks up each device's address once, with
// that device current, and passes that.  Every call on one device shares the
// array, so calls that may run at the same time on one device race.  The
// partials are written in full before they are read, so nothing needs
// clearing between calls.
static __device__ __align__(256) float scratch[kStepScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;

hipError_t step_scratch(int dev, float **out) {
    static std::mutex mu;
    static float *addr[kMaxDevices] = {};
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t back = hipSetDevice(cur);
            if (e == hipSuccess) e = back;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = static_cast<float *>(p);
    }
    *out = addr[dev];
    return hipSuccess;
}

hipError_t launch_step(const StepArgs &a, int io_bf16, hipStream_t s) {
    const dim3 block(NTH);
    if (a.nb > 1) {
        const long nblk = (long)a.BH * a.nb;
        const dim3 grid((unsigned)(nblk < kStepGrid ? nblk : kStepGrid));
        // (the initial state is given or not: a template argument, so that no
        // branch joins the memory's loads before their use)
        if (io_bf16 && a.C_in)
            hipLaunchKernelGGL((mlstm_step_rows_kernel<bf16, true>), grid, block, 0, s, a);
        else if (io_bf16)
            hipLaunchKernelGGL((mlstm_step_rows_kernel<bf16, false>), grid, block, 0, s, a);
        else if (a.C_in)
            hipLaunchKernelGGL((mlstm_step_rows_kernel<float, true>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((mlstm_step_rows_kernel<float, false>), grid, block, 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (io_bf16)
            hipLaunchKernelGGL(mlstm_step_finish_kernel<bf16>, dim3(a.BH), dim3(128), 0, s, a);
        else
            hipLaunchKernelGGL(mlstm_step_finish_kernel<float>, dim3(a.BH), dim3(128), 0, s, a);
    } else {
        const dim3 grid(a.BH);
        if (io_bf16)
            hipLaunchKernelGGL(mlstm_step_kernel<bf16>, grid, block, 0, s, a);
        else
            hipLaunchKernelGGL(mlstm_step_kernel<float>, grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace mlstm
