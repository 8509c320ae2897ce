// prefill_bf16.hpp -- chunkwise mLSTM forward for bf16 I/O on gfx950.
//
// Same mathematics as prefill_kernel.hpp (the chunkwise form of the xLSTM
// note's mLSTM recurrence, "mLSTM (matrix LSTM)" section, with the
// stabilizer of its "sLSTM" section): per chunk of L tokens, with
// b = in-chunk cumsum of f~, u_j = i~_j - b_j, r_i = max(m, max_{j<=i} u_j),
//   h_i = sigmoid(o~_i) (sum_j P_ij v_j + e^{m-r_i} C'^T q_i)
//                       / max(|sum_j P_ij + e^{m-r_i} n'.q_i|, e^{-(b_i+r_i)}),
//   P_ij = (q_i.k_j) e^{u_j - r_i} (j <= i),
//   C' <- e^{m-r_L} C' + sum_j e^{u_j-r_L} k_j v_j^T, n' likewise, m <- b_L + r_L.
//
// Schedule (one workgroup = one (pair, segment, BV value columns), 8
// wavefronts, two per SIMD so one can issue MFMAs while the other does
// VALU/LDS work):
//  * wavefront w = (p, hf): p = w & 3 owns BV/4 value columns, hf = w >> 2
//    owns half of the d_qk rows of the state C' (float32, registers, MFMA
//    accumulator layout).  The read-out C'^T Q^T is split over the two
//    halves (split-K) and the partial sums are exchanged through LDS; each
//    wavefront of the pair then finishes half of the chunk's token tiles;
//  * Q, K, V are staged with global->LDS copies (16 B per lane) into
//    row-major tiles whose 16-byte granules are XOR-swizzled per row; each
//    copy is issued after the last read of the buffer it refills within the
//    chunk (K is double buffered), so it lands while the rest of the chunk
//    and the start of the next one compute;
//  * K^T and V^T fragments (token index along the MFMA k) come from the LDS
//    transpose read (ds_read_b64_tr_b16) of the row-major tiles;
//  * the read-out splits C' into a bf16 high part and a bf16 remainder (two
//    MFMAs), so the carried state keeps ~16 significant bits in it;
//  * the decay of the carried state is applied lazily: C' is held as
//    C'/sigma and sigma (a product of per-chunk decays) is folded into the
//    read-out scale and the update weights, renormalised when it gets small;
//  * gate quantities of the next chunk are computed by one wavefront with
//    DPP scans into a double-buffered table; q.n' is a small VALU dot
//    product spread over all threads; n' is updated with MFMAs;
//  * two workgroup barriers per chunk, ordering LDS only, so copies stay in
//    flight across them.
// This schedule needs d_qk in {64, 128, 256} and d_v a multiple of BV; other
// shapes use the general kernel of prefill_kernel.hpp.
#pragma once

#include "prefill_kernel.hpp"

namespace mlstm {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

template <int L_, int DKP_, int BV_>
struct Bf16Cfg {
    static constexpr int L = L_, DKP = DKP_, BV = BV_;
    static constexpr int NW = 8, NTH = 512;
    static constexpr int LP = L < 32 ? 32 : L;        // token rows held (MFMA k of 32)
    static constexpr int NT = L / 16;                 // 16-token tiles per chunk
    static constexpr int NCT = NT * (NT + 1) / 2;     // causal tiles of S
    static constexpr int MYT = (NCT + NW - 1) / NW;   // S tiles per wavefront (max)
    static constexpr int NAT = DKP / 16;              // 16-row tiles of C'
    static constexpr int NAH = NAT / 2;               // ... per d_qk half
    static constexpr int NKS = DKP / 32, NKH = NKS / 2;
    static constexpr int NJS = LP / 32;
    static constexpr int WC = BV / 4;                 // value columns per wavefront pair
    static constexpr int NBT = WC / 16;
    static constexpr int NF = NT >= 2 ? NT / 2 : 1;   // token tiles each wavefront finishes
    static constexpr int QG = DKP / 8, VG = BV / 8, PG = LP / 8;  // granules per row
    static constexpr int NNW = (NAH + 3) / 4;         // n' tiles per wavefront (max)
    static constexpr int GT_FLOATS = 5 * LP + LP + 8; // u r s floor w | w hi/lo (bf16 pairs) | scalars
    static constexpr size_t LDS_BYTES =
        2 * ((size_t)LP * DKP * 3 + (size_t)LP * BV + (size_t)L * LP) +
        16 * (size_t)NW * NF * NBT * 64 + 4 * (2 * (size_t)GT_FLOATS + NCT * 16 + L + DKP) + 16;
    static_assert(QG >= 8 && VG >= 8, "swizzle needs 8 granules per row");
    static_assert(NBT >= 1 && WC % 16 == 0, "whole 16-column tiles per wavefront");
    static_assert(NKH >= 1, "d_qk split in two halves");
    static_assert(L <= 64, "one token per lane in the gate scan");
};

// row swizzle of the 16-byte granules (XOR within aligned groups of 8)
__device__ __forceinline__ int swz8(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }
template <int GPR>
__device__ __forceinline__ int swzg(int row) { return GPR >= 8 ? swz8(row) : (swz8(row) & (GPR - 1)); }
// element offset of (row, col) in a swizzled row-major bf16 tile with GPR granules per row
template <int GPR>
__device__ __forceinline__ int sw_off(int row, int col) {
    return row * GPR * 8 + (((col >> 3) ^ swzg<GPR>(row)) << 3) + (col & 7);
}

__device__ __forceinline__ bf16x4 tr_read(const bf16 *p) {
    s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
    return __builtin_bit_cast(bf16x4, r);
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x4 ld4(const bf16 *p) { return *reinterpret_cast<const bf16x4 *>(p); }

// split 8 floats into bf16 high parts and bf16 remainders
__device__ __forceinline__ void split8(const float *x, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bf16 h = (bf16)x[e];
        hi[e] = h;
        lo[e] = (bf16)(x[e] - (float)h);
    }
}

// inclusive scans over the 64 lanes of a wavefront with DPP: shifts of 1, 2,
// 4, 8 inside each row of 16 lanes, then the row totals carried forward with
// the row broadcasts of lane 15 and lane 31.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_mov(float identity, float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(x), CTRL,
                                                      ROWMASK, 0xf, false));
}
__device__ __forceinline__ float wave_scan_add(float x) {
    x += dpp_mov<0x111, 0xf>(0.0f, x);  // row_shr:1
    x += dpp_mov<0x112, 0xf>(0.0f, x);  // row_shr:2
    x += dpp_mov<0x114, 0xf>(0.0f, x);  // row_shr:4
    x += dpp_mov<0x118, 0xf>(0.0f, x);  // row_shr:8
    x += dpp_mov<0x142, 0xa>(0.0f, x);  // row_bcast:15 into rows 1, 3
    x += dpp_mov<0x143, 0xc>(0.0f, x);  // row_bcast:31 into rows 2, 3
    return x;
}
__device__ __forceinline__ float wave_scan_max(float x) {
    const float ni = -INFINITY;
    x = fmaxf(x, dpp_mov<0x111, 0xf>(ni, x));
    x = fmaxf(x, dpp_mov<0x112, 0xf>(ni, x));
    x = fmaxf(x, dpp_mov<0x114, 0xf>(ni, x));
    x = fmaxf(x, dpp_mov<0x118, 0xf>(ni, x));
    x = fmaxf(x, dpp_mov<0x142, 0xa>(ni, x));
    x = fmaxf(x, dpp_mov<0x143, 0xc>(ni, x));
    return x;
}

// Workgroup barrier for LDS data: this wavefront's LDS writes are complete
// (lgkmcnt 0) and at most VM of its vector-memory operations are still
// outstanding (they complete in issue order), so every global->LDS copy
// issued before the last VM of them has landed for all wavefronts after the
// barrier.  Copies issued later stay in flight across it.  The signal fences
// keep the compiler from moving LDS accesses across the barrier.
template <int VM>
__device__ __forceinline__ void block_sync() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 0xf) | (0x7 << 4) | (0x0 << 8) | ((VM >> 4) << 14));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait until at most VM of this wavefront's vector-memory operations are
// outstanding (no LDS wait).  Placed before the use of a plain load's result
// whose exact position in the issue order is known, so that the compiler does
// not add a full drain of the global->LDS copies issued after it.
template <int VM>
__device__ __forceinline__ void vm_wait() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 0xf) | (0x7 << 4) | (0xf << 8) | ((VM >> 4) << 14));
}

template <int L, int DKP, int BV, bool STATE_ONLY>
__global__ __launch_bounds__(512, 1) void mlstm_bf16_kernel(FwdArgs a) {
    using Cfg = Bf16Cfg<L, DKP, BV>;
    constexpr int NW = Cfg::NW, NTH = Cfg::NTH, LP = Cfg::LP, NT = Cfg::NT, NCT = Cfg::NCT;
    constexpr int MYT = Cfg::MYT, NAH = Cfg::NAH, NKH = Cfg::NKH, NJS = Cfg::NJS;
    constexpr int WC = Cfg::WC, NBT = Cfg::NBT, NF = Cfg::NF, QG = Cfg::QG, VG = Cfg::VG;
    constexpr int PG = Cfg::PG, NNW = Cfg::NNW, GTF = Cfg::GT_FLOATS;
    constexpr float kRenorm = 8.6736174e-19f;  // 2^-60: renormalise the lazy state scale below this

    __shared__ __attribute__((aligned(16))) bf16 Qs[LP * DKP];
    __shared__ __attribute__((aligned(16))) bf16 Ks[2][LP * DKP];  // K of even / odd chunks
    __shared__ __attribute__((aligned(16))) bf16 Vs[LP * BV];
    __shared__ __attribute__((aligned(16))) bf16 Ps[L * LP];
    __shared__ __attribute__((aligned(16))) f32x4 Xch[NW][NF * NBT][64];
    // gate tables (double buffered): u, r, s, floor, w [LP] floats, w as bf16
    // high/low pairs [LP], then scalars (m after, decay, sum f~)
    __shared__ __attribute__((aligned(16))) float gt[2][GTF];
    __shared__ float den_part[NCT * 16];
    __shared__ float qn[L];
    __shared__ __attribute__((aligned(16))) float nsh[DKP];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int p = wave & 3, hf = wave >> 2;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int te = l16 >> 2, tq = l16 & 3;  // transpose-read source row / column quad

    const int nwg = gridDim.x;
    int logical = blockIdx.x;
    if ((nwg & 7) == 0) logical = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
    const int gseg = STATE_ONLY ? a.nseg - 1 : a.nseg;
    const int tile = logical % a.ntile;
    const int rest = logical / a.ntile;
    const int seg = rest % gseg;
    const int bh = rest / gseg;

    const int dk = a.dk, dv = a.dv, T = a.T;  // here dk == DKP and dv is a multiple of BV
    const int t_begin = seg * a.seg_len;
    const int t_end = min(t_begin + a.seg_len, T);
    const int nchunks = (t_end - t_begin + L - 1) / L;
    const int col0 = tile * BV;
    const int wc0 = p * WC;  // first column of this wavefront pair (tile-local)

    const bf16 *qg = static_cast<const bf16 *>(a.q) + (size_t)bh * T * DKP;
    const bf16 *kg = static_cast<const bf16 *>(a.k) + (size_t)bh * T * DKP;
    const bf16 *vg = static_cast<const bf16 *>(a.v) + (size_t)bh * T * dv + col0;
    const bf16 *og = static_cast<const bf16 *>(a.o) + (size_t)bh * T * dv + col0;
    bf16 *hg = static_cast<bf16 *>(a.h) + (size_t)bh * T * dv + col0;
    const float *igg = a.ig + (size_t)bh * T;
    const float *fgg = a.fg + (size_t)bh * T;

    // ---- zero every tile once: padding rows and P's upper tiles stay zero
    {
        const uint4 z = make_uint4(0, 0, 0, 0);
        uint4 *q4 = reinterpret_cast<uint4 *>(Qs);
        for (int e = tid; e < LP * DKP / 8; e += NTH) q4[e] = z;
        uint4 *k4 = reinterpret_cast<uint4 *>(&Ks[0][0]);
        for (int e = tid; e < 2 * LP * DKP / 8; e += NTH) k4[e] = z;
        uint4 *v4 = reinterpret_cast<uint4 *>(Vs);
        for (int e = tid; e < LP * BV / 8; e += NTH) v4[e] = z;
        uint4 *p4 = reinterpret_cast<uint4 *>(Ps);
        for (int e = tid; e < L * LP / 8; e += NTH) p4[e] = z;
        for (int e = tid; e < 2 * GTF; e += NTH) (&gt[0][0])[e] = 0.0f;
    }

    // ---- initial state (C' rows of this wavefront's d_qk half, its pair's columns)
    const size_t rec = seg_state_floats(dk, dv);
    const float *Cs = nullptr, *ns = nullptr;
    float m_prev = 0.0f;
    if (STATE_ONLY) {
        m_prev = -1e30f;  // "no past": the first chunk's stabilizer comes from its own gates
    } else if (a.seg_in) {
        const float *r = a.seg_in + ((size_t)bh * a.nseg + seg) * rec;
        Cs = r;
        ns = r + (size_t)dk * dv;
        m_prev = r[(size_t)dk * dv + dk];
    } else if (a.C0) {
        Cs = a.C0 + (size_t)bh * dk * dv;
        ns = a.n0 + (size_t)bh * dk;
        m_prev = a.m0[bh];
    }
    const int arow0 = hf * (DKP / 2);  // first d_qk row of this wavefront's half
    const int bcol = col0 + wc0 + l16; // state column of this lane (tile bt adds 16 bt)
    f32x4 Cr[NAH][NBT];
#pragma unroll
    for (int at = 0; at < NAH; ++at)
#pragma unroll
        for (int bt = 0; bt < NBT; ++bt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Cr[at][bt][r] = Cs ? Cs[(size_t)(arow0 + 16 * at + 4 * g4 + r) * dv + bcol + 16 * bt] : 0.0f;
    // n' lives in LDS (true scale); 16-row tiles p + 4x of each half are
    // updated by the wavefront (p, hf) with an MFMA whose column 0 is K^T w
    for (int e = tid; e < DKP; e += NTH) nsh[e] = ns ? ns[e] : 0.0f;
    float sigma = 1.0f;  // C' is held divided by sigma

    // ---- global -> LDS copies, fully unrolled.  Physical granule g of a tile
    // is (row, gl) with gl = (g % gpr) ^ swz(row); each lane of a copy
    // instruction fetches the granule that belongs at its LDS slot.  Rows past
    // the segment end are clamped to its last row (finite data; their gates
    // zero them out).
    // Instruction k of a wavefront fills granules [(k NW + wave) 64, +64), i.e.
    // rows row0 + k RPI with RPI = NW 64 / GPR a multiple of 8, so the swizzle
    // of a lane is the same for every k: the per-lane part of the address is
    // one byte offset (voff), the rest is uniform.
    // (recomputed at every copy from an opaque copy of the lane index, so the
    // compiler does not keep it live across the chunk loop)
    auto lane_voff = [&](auto gpr_c, int ld) -> int {
        constexpr int GPR = decltype(gpr_c)::value;
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int pgr = wave * 64 + ln;
        const int row = pgr / GPR;
        const int gl = (pgr % GPR) ^ swz8(row);
        return row * ld * 2 + gl * 16;
    };
    auto copy_tile = [&](bf16 *dst, const bf16 *src, int ld, auto gpr_c, int tc) {
        constexpr int GPR = decltype(gpr_c)::value;
        const int voff = lane_voff(gpr_c, ld);
        constexpr int TOTAL = L * GPR;                    // granules
        constexpr int NI = (TOTAL + NW * 64 - 1) / (NW * 64);
        constexpr int RPI = NW * 64 / GPR;
        static_assert(RPI % 8 == 0, "rows per copy instruction keep the swizzle");
        if (tc + L <= t_end) {  // whole chunk inside the segment
#pragma unroll
            for (int k = 0; k < NI; ++k) {
                const int blk = (k * NW + wave) * 64;
                if (TOTAL % (NW * 64) == 0 || blk < TOTAL) {
                    const char *base = reinterpret_cast<const char *>(src + (size_t)(tc + k * RPI) * ld);
                    __builtin_amdgcn_global_load_lds((const void *)(base + voff), (lds_void *)(dst + blk * 8),
                                                     16, 0, 0);
                }
            }
        } else {  // last chunk of the segment: rows past its end read its last row
            // (same instruction count as above, so waits on later copies stay exact)
            int ln = lane;
            asm volatile("" : "+v"(ln));
#pragma unroll
            for (int k = 0; k < NI; ++k) {
                const int blk = (k * NW + wave) * 64;
                if (TOTAL % (NW * 64) == 0 || blk < TOTAL) {
                    const int pgr = blk + ln;
                    const int row = pgr / GPR;
                    const int gl = (pgr % GPR) ^ swz8(row);
                    const int t = min(tc + row, t_end - 1);
                    __builtin_amdgcn_global_load_lds((const void *)(src + (size_t)t * ld + gl * 8),
                                                     (lds_void *)(dst + blk * 8), 16, 0, 0);
                }
            }
        }
    };
    using QGc = std::integral_constant<int, QG>;
    using VGc = std::integral_constant<int, VG>;

    // ---- gates (wavefront GW; one token per lane)
    constexpr int GW = NW - 1;
    // raw loads here; lanes past the segment are masked in gate_prep, so the
    // loads stay in flight until then
    float gf = 0.0f, gi = -INFINITY;
    bool gok = false;
    auto load_gates = [&](int c) {
        const int t = t_begin + c * L + lane;
        gok = lane < L && t < t_end;
        const int tc = min(t, t_end - 1);
        gf = fgg[tc];
        gi = igg[tc];
    };
    auto gate_prep = [&](float m_before, float *G) {
        const float b = wave_scan_add(gok ? gf : 0.0f);
        const float u = (gok ? gi : -INFINITY) - b;
        const float pm = wave_scan_max(u);
        const float r = fmaxf(m_before, pm);
        const float r_last = __shfl(r, L - 1, 64);
        const float b_last = __shfl(b, L - 1, 64);
        if (lane < L) {
            const float w = exp_e(u - r_last);
            G[lane] = u;
            G[LP + lane] = r;
            G[2 * LP + lane] = exp_e(m_before - r);
            G[3 * LP + lane] = exp_e(-(b + r));
            G[4 * LP + lane] = w;
            const bf16 whi = (bf16)w;
            const bf16 wlo = (bf16)(w - (float)whi);
            bf16 *W2 = reinterpret_cast<bf16 *>(&G[5 * LP]);
            W2[lane] = whi;
            W2[LP + lane] = wlo;
        }
        if (lane == 0) {
            G[6 * LP + 0] = b_last + r_last;          // stabilizer after the chunk
            G[6 * LP + 1] = exp_e(m_before - r_last); // decay of the carried state
            G[6 * LP + 2] = b_last;                   // sum of the chunk's log forget gates
        }
    };

    // ---- causal S tiles of this wavefront: t = wave + NW x
    int tjt[MYT], tit[MYT];
    bool tok[MYT];
#pragma unroll
    for (int x = 0; x < MYT; ++x) {
        const int t = wave + NW * x;
        tok[x] = t < NCT;
        int it = 0;
        while ((it + 1) * (it + 2) / 2 <= t) ++it;
        tit[x] = it;
        tjt[x] = t - it * (it + 1) / 2;
    }
    // token tiles of the read-out in slot order: this wavefront's own tiles
    // first (it finishes them), then the partner's (it hands their partial
    // sums over).  NT = 4: tiles {0, 3} and {1, 2} (balanced causal work).
    const int nown = (NT == 1 && hf == 1) ? 0 : NF;
    int slot_it[NT];
    if constexpr (NT == 4) {
        slot_it[0] = hf;
        slot_it[1] = 3 - hf;
        slot_it[2] = 1 - hf;
        slot_it[3] = 2 + hf;
    } else if constexpr (NT == 2) {
        slot_it[0] = hf;
        slot_it[1] = 1 - hf;
    } else {
        slot_it[0] = 0;
    }
    // own slot f needs the k-step js of V^T P^T (P is zero above the diagonal):
    // with NT = 4 the first own tile is 0 or 1 (one k-step), the second 2 or 3
    auto need_js = [](int f, int js) constexpr { return js == 0 || (NT == 4 && f == 1); };

    // ---- per-lane LDS offsets (loop invariant)
    const int s16 = swz8(l16);  // swizzle of rows 16 t + l16
    // Q / K fragment for k-step ks: rows 16 t + l16, columns 32 ks + 4 g4 (+16)
    int qkoff[2][2];
#pragma unroll
    for (int par = 0; par < 2; ++par)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            qkoff[par][hh] = l16 * DKP + (((((par << 2) | ((g4 >> 1) + 2 * hh)) ^ s16)) << 3) + 4 * (g4 & 1);
    auto qk_frag = [&](const bf16 *tilebase, int ks) -> bf16x8 {  // tilebase: row 16 t of the tile
        const bf16 *b = tilebase + ((ks >> 1) << 6);
        return cat8(ld4(b + qkoff[ks & 1][0]), ld4(b + qkoff[ks & 1][1]));
    };
    // transpose reads: rows 32 js + 8 g4 + te (+4), columns c0 + 4 tq
    const int trow0 = 8 * g4 + te, trow1 = trow0 + 4;
    auto tr_frag = [&](const bf16 *rowblock, auto gpr_c, int c0) -> bf16x8 {
        constexpr int GPR = decltype(gpr_c)::value;
        return cat8(tr_read(rowblock + sw_off<GPR>(trow0, c0)), tr_read(rowblock + sw_off<GPR>(trow1, c0)));
    };

    float g_total = 0.0f;
    if (nchunks > 0) {
        block_sync<0>();  // zeroing done before the copies land
        if (!STATE_ONLY) copy_tile(Qs, qg, DKP, QGc{}, t_begin);
        copy_tile(Ks[0], kg, DKP, QGc{}, t_begin);
        copy_tile(Vs, vg, dv, VGc{}, t_begin);
        if (wave == GW) {
            load_gates(0);
            vm_wait<0>();
            gate_prep(m_prev, gt[0]);
        }
    }
    block_sync<0>();

    // Pipeline of the copies (each fills a buffer no wavefront reads until a
    // later barrier):
    //   after the S tiles of chunk c   K(c+1) -> the other K buffer (read
    //                                  last in chunk c-1)
    //   after barrier C                Q(c+1) (every wavefront is done with Q(c))
    //   after barrier D                V(c+1) (first read after barrier C of c+1)
    // Barrier C waits for V(c), barrier D for Q(c+1) and K(c+1).
    constexpr int NIK = (L * QG) / (NW * 64);          // K (and Q) copy instructions per wavefront
    constexpr bool EXACT = (L * QG) % (NW * 64) == 0 && NT >= 2;
    constexpr int NORW = NF * NBT;                      // output-gate loads after the K copy
    constexpr int VM_C = EXACT ? NIK + NORW : 0;        // outstanding allowed at barrier C
    constexpr int VM_D = EXACT ? NF * NBT : 0;          // ... at barrier D (this chunk's h stores)
    for (int c = 0; c < nchunks; ++c) {
        const bf16 *K = Ks[c & 1];
        bf16 *Knext = Ks[(c + 1) & 1];
        const float *G = gt[c & 1];
        float *Gnext = gt[(c + 1) & 1];
        const int tc = t_begin + c * L;
        const float m_next = G[6 * LP + 0], s_last = G[6 * LP + 1];
        g_total += G[6 * LP + 2];
        const bool more = c + 1 < nchunks;

        uint2 orw[NF][NBT];  // output-gate inputs of this wavefront's own tiles
        if (more && wave == GW) load_gates(c + 1);

        f32x4 Ot[NBT][NT];
        if (!STATE_ONLY) {
            // q.n' for every token (VALU, all threads), n' of the previous state
            {
                constexpr int PARTS = NTH / L;
                constexpr int SPAN = DKP / PARTS;  // >= 2
                const int i = tid / PARTS, part = tid % PARTS;
                float acc = 0.0f;
                if constexpr (SPAN >= 8) {
#pragma unroll
                    for (int e = 0; e < SPAN / 8; ++e) {
                        const int col = part * SPAN + 8 * e;
                        const bf16x8 qv = *reinterpret_cast<const bf16x8 *>(&Qs[sw_off<QG>(i, col)]);
                        const f32x4 n0 = *reinterpret_cast<const f32x4 *>(&nsh[col]);
                        const f32x4 n1 = *reinterpret_cast<const f32x4 *>(&nsh[col + 4]);
#pragma unroll
                        for (int x = 0; x < 4; ++x) {
                            acc = fmaf((float)qv[x], n0[x], acc);
                            acc = fmaf((float)qv[x + 4], n1[x], acc);
                        }
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < SPAN; ++e) {
                        const int col = part * SPAN + e;
                        acc = fmaf((float)Qs[sw_off<QG>(i, col)], nsh[col], acc);
                    }
                }
#pragma unroll
                for (int off = 1; off < PARTS && off < 64; off <<= 1) acc += __shfl_xor(acc, off, 64);
                if (part == 0) qn[i] = acc;
            }

            __builtin_amdgcn_sched_barrier(0);
            // causal S tiles over all of d_qk (next k-step's fragments fetched ahead)
            f32x4 St[MYT];
#pragma unroll
            for (int x = 0; x < MYT; ++x) {
                St[x] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (tok[x]) {
                    const bf16 *q0 = Qs + 16 * tit[x] * DKP;
                    const bf16 *k0 = K + 16 * tjt[x] * DKP;
                    bf16x8 fq = qk_frag(q0, 0), fk = qk_frag(k0, 0);
#pragma unroll
                    for (int ks = 0; ks < 2 * NKH; ++ks) {
                        bf16x8 nq, nk;
                        if (ks + 1 < 2 * NKH) {
                            nq = qk_frag(q0, ks + 1);
                            nk = qk_frag(k0, ks + 1);
                        }
                        St[x] = mfma(fk, fq, St[x]);
                        if (ks + 1 < 2 * NKH) {
                            fq = nq;
                            fk = nk;
                        }
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            // K(c) is not read again until the state update: fetch K(c+1)
            if (more) copy_tile(Knext, kg, DKP, QGc{}, tc + L);
            // next chunk's gate table (one wavefront)
            if (more && wave == GW) {
                vm_wait<EXACT ? NIK : 0>();  // gate loads were issued before the K copy
                gate_prep(m_next, Gnext);
            }

            // P = S (x) e^{u_j - r_i} -> LDS (bf16); column sums -> den_part
#pragma unroll
            for (int x = 0; x < MYT; ++x) {
                if (tok[x]) {
                    const int i = 16 * tit[x] + l16;
                    const float ri = G[LP + i];
                    float pv[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 16 * tjt[x] + 4 * g4 + r;
                        pv[r] = (j <= i) ? St[x][r] * exp_e(G[j] - ri) : 0.0f;
                    }
                    const bf16x4 pb = {(bf16)pv[0], (bf16)pv[1], (bf16)pv[2], (bf16)pv[3]};
                    *reinterpret_cast<bf16x4 *>(&Ps[sw_off<PG>(i, 16 * tjt[x] + 4 * g4)]) = pb;
                    float cs = (pv[0] + pv[1]) + (pv[2] + pv[3]);
                    cs += __shfl_xor(cs, 16, 64);
                    cs += __shfl_xor(cs, 32, 64);
                    if (g4 == 0) den_part[(wave + NW * x) * 16 + l16] = cs;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            // O^T partial over this half of d_qk: C'^T Q^T, C' split into hi + lo.
            // Q fragments of the next k-step are fetched before this one's MFMAs.
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt)
#pragma unroll
                for (int s = 0; s < NT; ++s) Ot[bt][s] = f32x4{0.f, 0.f, 0.f, 0.f};
            const bf16 *qrow[NT];
#pragma unroll
            for (int s = 0; s < NT; ++s) qrow[s] = Qs + 16 * slot_it[s] * DKP;
            bf16x8 bq = qk_frag(qrow[0], hf * NKH);
#pragma unroll
            for (int kk = 0; kk < NKH; ++kk) {
                bf16x8 ach[NBT], acl[NBT];
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt) {
                    const float x[8] = {Cr[2 * kk][bt][0], Cr[2 * kk][bt][1], Cr[2 * kk][bt][2],
                                        Cr[2 * kk][bt][3], Cr[2 * kk + 1][bt][0], Cr[2 * kk + 1][bt][1],
                                        Cr[2 * kk + 1][bt][2], Cr[2 * kk + 1][bt][3]};
                    split8(x, ach[bt], acl[bt]);
                }
#pragma unroll
                for (int s = 0; s < NT; ++s) {
                    bf16x8 bqn;
                    const bool nxt = s + 1 < NT || kk + 1 < NKH;
                    if (nxt) bqn = qk_frag(qrow[(s + 1) % NT], hf * NKH + kk + (s + 1) / NT);
#pragma unroll
                    for (int bt = 0; bt < NBT; ++bt) {
                        Ot[bt][s] = mfma(ach[bt], bq, Ot[bt][s]);
                        Ot[bt][s] = mfma(acl[bt], bq, Ot[bt][s]);
                    }
                    if (nxt) bq = bqn;
                }
            }
            // hand the partner the partial sums of the tiles it finishes
#pragma unroll
            for (int s = 0; s < NT; ++s) {
                if (s >= nown) {
#pragma unroll
                    for (int bt = 0; bt < NBT; ++bt) Xch[wave ^ 4][(s - nown) * NBT + bt][lane] = Ot[bt][s];
                }
            }
#pragma unroll
            for (int f = 0; f < NF; ++f)
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt) {
                    const int t = min(tc + 16 * slot_it[f] + l16, t_end - 1);
                    orw[f][bt] = *reinterpret_cast<const uint2 *>(og + (size_t)t * dv + wc0 + 16 * bt + 4 * g4);
                }
        } else {
            if (more) copy_tile(Knext, kg, DKP, QGc{}, tc + L);
            if (more && wave == GW) {
                vm_wait<EXACT ? NIK : 0>();  // gate loads were issued before the K copy
                gate_prep(m_next, Gnext);
            }
        }
        // (C) V(c) landed; P, den_part, qn, Xch visible; Q(c) free.  The last
        // chunk issued no K copy, so only the output-gate loads may stay.
        if (more)
            block_sync<STATE_ONLY ? 0 : VM_C>();
        else
            block_sync<(STATE_ONLY || !EXACT) ? 0 : NORW>();
        if (more && !STATE_ONLY) copy_tile(Qs, qg, DKP, QGc{}, tc + L);
        // output-gate loads (issued before barrier C) complete; Q(c+1) stays in flight
        if (!STATE_ONLY) {
            if (more)
                vm_wait<EXACT ? NIK : 0>();
            else
                vm_wait<0>();
        }

        if (!STATE_ONLY) {
            // finish this wavefront's own token tiles: partner's partial,
            // inter-chunk scale, V^T P^T, normaliser, output gate
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                __builtin_amdgcn_sched_barrier(0);
                if (f >= nown) continue;
                const int it = slot_it[f];
                const int i = 16 * it + l16;
                const float si = G[2 * LP + i] * sigma;
                f32x4 acc[NBT];
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt) acc[bt] = (Ot[bt][f] + Xch[wave][f * NBT + bt][lane]) * si;
                // O^T += V^T P^T (fragments loaded next to their use: low register pressure;
                // the other wavefront on the SIMD covers the LDS latency)
#pragma unroll
                for (int js = 0; js < NJS; ++js) {
                    if (need_js(f, js)) {
                        const bf16x8 bp = *reinterpret_cast<const bf16x8 *>(&Ps[sw_off<PG>(i, 32 * js + 8 * g4)]);
#pragma unroll
                        for (int bt = 0; bt < NBT; ++bt)
                            acc[bt] = mfma(tr_frag(Vs + 32 * js * BV, VGc{}, wc0 + 16 * bt + 4 * tq), bp, acc[bt]);
                    }
                }
                float den = G[2 * LP + i] * qn[i];
                // column tiles jt <= it contribute; every index below stays inside den_part
#pragma unroll
                for (int jt = 0; jt < NT; ++jt) {
                    const float dp = den_part[(it * (it + 1) / 2 + jt) * 16 + l16];
                    den += jt <= it ? dp : 0.0f;
                }
                const float inv = __builtin_amdgcn_rcpf(fmaxf(fabsf(den), G[3 * LP + i]));
                const int t = tc + i;
                if (t < t_end) {
#pragma unroll
                    for (int bt = 0; bt < NBT; ++bt) {
                        const uint2 o4 = orw[f][bt];
                        float y[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t wd = e < 2 ? o4.x : o4.y;
                            const float ox = __uint_as_float((e & 1) ? (wd & 0xffff0000u) : (wd << 16));
                            y[e] = acc[bt][e] * inv * __builtin_amdgcn_rcpf(1.0f + exp_e(-ox));
                        }
                        const bf16x4 hv = {(bf16)y[0], (bf16)y[1], (bf16)y[2], (bf16)y[3]};
                        *reinterpret_cast<bf16x4 *>(hg + (size_t)t * dv + wc0 + 16 * bt + 4 * g4) = hv;
                    }
                }
            }
        }

        __builtin_amdgcn_sched_barrier(0);
        // ---- C'/sigma += K^T ((w/sigma') (x) V),  n'/sigma likewise  (sigma' = sigma * decay)
        sigma *= s_last;
        if (sigma < kRenorm) {  // uniform: fold sigma back into the held state
#pragma unroll
            for (int at = 0; at < NAH; ++at)
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt) Cr[at][bt] *= sigma;
            sigma = 1.0f;
        }
        const float rsig = __builtin_amdgcn_rcpf(sigma);
        f32x4 nacc[NNW];  // K^T w for this wavefront's n' tiles (column 0)
#pragma unroll
        for (int x = 0; x < NNW; ++x) nacc[x] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int js = 0; js < NJS; ++js) {
            const bf16 *k0 = K + 32 * js * DKP;
            // K^T fragments in groups of 4 d_qk tiles, the next group fetched ahead
            constexpr int GRP = 2;  // NAH is even
            bf16x8 ak[GRP];
#pragma unroll
            for (int u = 0; u < GRP; ++u) ak[u] = tr_frag(k0, QGc{}, arow0 + 16 * u + 4 * tq);
            float w8[8];
            {
                const f32x4 w0 = *reinterpret_cast<const f32x4 *>(&G[4 * LP + 32 * js + 8 * g4]);
                const f32x4 w1 = *reinterpret_cast<const f32x4 *>(&G[4 * LP + 32 * js + 8 * g4 + 4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    w8[e] = w0[e] * rsig;
                    w8[e + 4] = w1[e] * rsig;
                }
            }
            bf16x8 bw[NBT];
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt) {
                const bf16x8 vv = tr_frag(Vs + 32 * js * BV, VGc{}, wc0 + 16 * bt + 4 * tq);
#pragma unroll
                for (int e = 0; e < 8; ++e) bw[bt][e] = (bf16)((float)vv[e] * w8[e]);
            }
            // w (hi, lo) as a 16-column operand with only column 0 non-zero (for n')
            bf16x8 bnh, bnl;
            {
                const bf16 *W2 = reinterpret_cast<const bf16 *>(&G[5 * LP]);
                const uint4 wh = *reinterpret_cast<const uint4 *>(W2 + 32 * js + 8 * g4);
                const uint4 wl = *reinterpret_cast<const uint4 *>(W2 + LP + 32 * js + 8 * g4);
                const bool c0 = l16 == 0;
                const uint4 zh = {c0 ? wh.x : 0u, c0 ? wh.y : 0u, c0 ? wh.z : 0u, c0 ? wh.w : 0u};
                const uint4 zl = {c0 ? wl.x : 0u, c0 ? wl.y : 0u, c0 ? wl.z : 0u, c0 ? wl.w : 0u};
                bnh = *reinterpret_cast<const bf16x8 *>(&zh);
                bnl = *reinterpret_cast<const bf16x8 *>(&zl);
            }
#pragma unroll
            for (int g0 = 0; g0 < NAH; g0 += GRP) {
                __builtin_amdgcn_sched_barrier(0);
                bf16x8 akn[GRP];
                if (g0 + GRP < NAH) {
#pragma unroll
                    for (int u = 0; u < GRP; ++u) akn[u] = tr_frag(k0, QGc{}, arow0 + 16 * (g0 + GRP + u) + 4 * tq);
                }
#pragma unroll
                for (int u = 0; u < GRP; ++u) {
                    const int at = g0 + u;
#pragma unroll
                    for (int bt = 0; bt < NBT; ++bt) Cr[at][bt] = mfma(ak[u], bw[bt], Cr[at][bt]);
#pragma unroll
                    for (int x = 0; x < NNW; ++x) {
                        if (at == p + 4 * x) {
                            nacc[x] = mfma(ak[u], bnh, nacc[x]);
                            nacc[x] = mfma(ak[u], bnl, nacc[x]);
                        }
                    }
                }
                if (g0 + GRP < NAH) {
#pragma unroll
                    for (int u = 0; u < GRP; ++u) ak[u] = akn[u];
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // n' <- decay n' + K^T w (this wavefront's tiles; read again after barrier D)
        if (l16 == 0) {
#pragma unroll
            for (int x = 0; x < NNW; ++x) {
                const int tl = p + 4 * x;
                if (tl < NAH) {
                    f32x4 *np = reinterpret_cast<f32x4 *>(&nsh[arow0 + 16 * tl + 4 * g4]);
                    *np = *np * s_last + nacc[x];
                }
            }
        }
        m_prev = m_next;
        block_sync<STATE_ONLY ? 0 : VM_D>();  // (D) Q(c+1), K(c+1) landed; n' visible; V(c) free
        if (more) copy_tile(Vs, vg, dv, VGc{}, tc + L);
    }

    // ---- state out
    float *Cdst = nullptr, *ndst = nullptr, *mdst = nullptr;
    if (STATE_ONLY) {
        float *r = a.seg_out + ((size_t)bh * (a.nseg - 1) + seg) * rec;
        Cdst = r;
        ndst = r + (size_t)dk * dv;
        mdst = ndst + dk;
        if (tile == 0 && tid == 0) mdst[1] = g_total;
    } else if (a.CT && seg == a.nseg - 1) {
        Cdst = a.CT + (size_t)bh * dk * dv;
        ndst = a.nT + (size_t)bh * dk;
        mdst = a.mT + bh;
    }
    if (Cdst) {
#pragma unroll
        for (int at = 0; at < NAH; ++at)
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Cdst[(size_t)(arow0 + 16 * at + 4 * g4 + r) * dv + bcol + 16 * bt] = Cr[at][bt][r] * sigma;
        if (tile == 0) {
            for (int e = tid; e < dk; e += NTH) ndst[e] = nsh[e];
            if (tid == 0) mdst[0] = m_prev;
        }
    }
}

}  // namespace mlstm
