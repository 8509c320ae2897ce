// prefill_kernel.hpp -- chunkwise-parallel mLSTM forward on gfx950 MFMA.
//
// The recurrence (xLSTM note: "sLSTM" section for the exponential gates and
// the stabilizer m_t = max(f~_t + m_{t-1}, i~_t), "mLSTM (matrix LSTM)"
// section for C_t = f_t C_{t-1} + i_t v_t k_t^T, n_t = f_t n_{t-1} + i_t k_t
// and h_t = o_t * C_t q_t / max(|n_t^T q_t|, 1)) is linear in (C, n), so a
// chunk of L tokens can be evaluated at once from the state before it.  The
// note only names the chunkwise schedule; the algebra below is derived by
// unrolling the recurrence inside a chunk.  With the in-chunk inclusive
// cumulative sum b_i = sum_{r<=i} f~_r, u_j = i~_j - b_j and m the stabilizer
// before the chunk:
//
//   r_i   = max(m, max_{j<=i} u_j)          M_i = b_i + r_i = m_t at token i
//   P_ij  = (q_i . k_j) e^{u_j - r_i}       (j <= i, else 0)
//   num_i = sum_j P_ij v_j + e^{m - r_i} C'^T q_i
//   den_i = sum_j P_ij      + e^{m - r_i} n'^T q_i
//   h_i   = sigmoid(o~_i) * num_i / max(|den_i|, e^{-M_i})
//
// and the state after the chunk (w_j = e^{u_j - r_{L-1}}):
//   C' <- e^{m - r_{L-1}} C' + sum_j w_j k_j v_j^T,   n' likewise with k_j,
//   m  <- b_{L-1} + r_{L-1}.
// Every exponent is <= 0, so nothing overflows however large i~ gets.
//
// Schedule.  One workgroup (NW wavefronts) owns one (pair, segment, block of
// BV value columns) and walks the chunks of its segment in order, keeping its
// d_qk x BV slice of C' in registers for the whole sequence; each wavefront
// owns BV/NW columns of it.  Per chunk:
//   S^T = K Q^T (only the causal 16x16 tiles, spread over the wavefronts),
//   O^T = C'^T Q^T, with C' converted to bf16 high-part and remainder
//         fragments straight from the MFMA accumulator layout (a
//         permutation of the k index that the Q and K fragments follow too),
//         so C' never goes through LDS;
//   P   = S (x) decay, shared through LDS as bf16;  O^T += V^T P^T;
//   h from O^T, the shared denominators and the output gate;
//   C'  = decay * C' + K^T (w (x) V)   (MFMA accumulating into the registers).
// Q, K, K^T, V^T and P of the chunk sit in LDS; K^T and V^T (the token index
// contiguous) are written transposed from registers when the chunk is staged.
// The next chunk's tiles are loaded into registers while the current chunk
// computes and are written to LDS after it.  All MFMAs are
// v_mfma_f32_16x16x32_bf16 with float32 accumulation.  For float32 I/O every
// operand is split into three bf16 parts (24 significant bits, as float32)
// and six MFMAs are issued per product (every part product above 2^-24 of
// it), so each product is float32-grade.  For bf16 I/O the read-out splits
// C' into a high part and a remainder against the exact bf16 q (two MFMAs);
// the other products take bf16 operands.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace mlstm {

template <typename IO, int L_, int DKP_, int BV_, int NW_>
struct PrefillCfg {
    static constexpr int L = L_, DKP = DKP_, BV = BV_, NW = NW_;
    static constexpr bool SPLIT = std::is_same<IO, float>::value;
    using TS = typename std::conditional<SPLIT, float, bf16>::type;  // LDS element
    static constexpr int NTH = 64 * NW;
    static constexpr int LP = L < 32 ? 32 : L;     // token extent padded to the MFMA k of 32
    static constexpr int NT = L / 16;              // 16-token tiles per chunk
    static constexpr int NCT = NT * (NT + 1) / 2;  // causal tiles of S
    static constexpr int MYT = (NCT + NW - 1) / NW;
    static constexpr int NAT = DKP / 16;           // 16-row tiles of C'
    static constexpr int NKS = DKP / 32;           // k-steps over d_qk
    static constexpr int NJS = LP / 32;            // k-steps over the chunk
    static constexpr int WC = BV / NW;             // value columns per wavefront
    static constexpr int NBT = WC / 16;
    static constexpr int QST = DKP + 4;            // row stride of Q, K tiles (elements)
    static constexpr int TST = LP + (SPLIT ? 4 : 8);  // row stride of K^T, V^T, P tiles
    static constexpr int VEC = 16 / (int)sizeof(IO);  // elements per 16-byte global load
    static constexpr int UQK = ((L / 4) * (DKP / VEC) + NTH - 1) / NTH;  // staging units/thread
    static constexpr int UV = ((L / 4) * (BV / VEC) + NTH - 1) / NTH;
    static constexpr size_t LDS_BYTES =
        sizeof(TS) * ((size_t)2 * L * QST + (size_t)DKP * TST + (size_t)BV * TST + (size_t)L * TST) +
        sizeof(float) * ((size_t)5 * LP + NCT * 16 + L + DKP + 4);
    static_assert(WC % 16 == 0, "a wavefront owns whole 16-column tiles");
    static_assert(NTH >= L, "one thread per token row at least");
    static_assert(L <= 64 || NW >= 1, "");
};

// ---------------------------------------------------------------- fragments
template <bool SPLIT> struct Frag;
template <> struct Frag<false> { bf16x8 x; };
// float32 operand as three bf16 parts: x = hi + mid + lo to about 2^-25 |x|
template <> struct Frag<true> { bf16x8 hi, mid, lo; };
// float32 state against an exact bf16 operand: high part and remainder
struct Frag2 { bf16x8 hi, lo; };

__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Frag<false> &a, const Frag<false> &b, f32x4 c) {
    return mfma(a.x, b.x, c);
}
// the six part products down to 2^-16 of the product (the three dropped ones,
// mid*lo, lo*mid and lo*lo, are below 2^-24 of it): float32-grade products,
// smallest terms first
__device__ __forceinline__ f32x4 mma(const Frag<true> &a, const Frag<true> &b, f32x4 c) {
    c = mfma(a.lo, b.hi, c);
    c = mfma(a.hi, b.lo, c);
    c = mfma(a.mid, b.mid, c);
    c = mfma(a.mid, b.hi, c);
    c = mfma(a.hi, b.mid, c);
    return mfma(a.hi, b.hi, c);
}
// the float32 state against an exact bf16 B operand
__device__ __forceinline__ f32x4 mma(const Frag2 &a, const Frag<false> &b, f32x4 c) {
    c = mfma(a.hi, b.x, c);
    return mfma(a.lo, b.x, c);
}

// 8 floats -> fragment (bf16, or bf16 high part + bf16 remainder)
__device__ __forceinline__ void set_frag(Frag<false> &f, const float *x) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f.x[e] = (bf16)x[e];
}
__device__ __forceinline__ void set_frag(Frag<true> &f, const float *x) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bf16 h = (bf16)x[e];
        const float r = x[e] - (float)h;  // exact
        const bf16 md = (bf16)r;
        f.hi[e] = h;
        f.mid[e] = md;
        f.lo[e] = (bf16)(r - (float)md);  // r - md exact
    }
}
__device__ __forceinline__ void set_frag(Frag2 &f, const float *x) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bf16 h = (bf16)x[e];
        f.hi[e] = h;
        f.lo[e] = (bf16)(x[e] - (float)h);
    }
}

// fragment whose 8 k-slots are two runs of 4 at p[0..3] and p[16..19]
__device__ __forceinline__ void load_frag_perm(Frag<false> &f, const bf16 *p) {
    bf16x4 a = *reinterpret_cast<const bf16x4 *>(p);
    bf16x4 b = *reinterpret_cast<const bf16x4 *>(p + 16);
    f.x = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void load_frag_perm(Frag<true> &f, const float *p) {
    f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    f32x4 b = *reinterpret_cast<const f32x4 *>(p + 16);
    float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    set_frag(f, x);
}
// fragment whose 8 k-slots are contiguous at p[0..7]
__device__ __forceinline__ void load_frag_nat(Frag<false> &f, const bf16 *p) {  // 16-byte aligned
    f.x = *reinterpret_cast<const bf16x8 *>(p);
}
__device__ __forceinline__ void load_frag_nat(Frag<true> &f, const float *p) {
    f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
    float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    set_frag(f, x);
}
// contiguous fragment with every k-slot scaled by w[e]
__device__ __forceinline__ void load_frag_nat_scaled(Frag<false> &f, const bf16 *p, const float *w) {
    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(p);
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)a[e] * w[e];
    set_frag(f, x);
}
__device__ __forceinline__ void load_frag_nat_scaled(Frag<true> &f, const float *p, const float *w) {
    f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[e] = a[e] * w[e];
        x[e + 4] = b[e] * w[e + 4];
    }
    set_frag(f, x);
}

// 4 consecutive LDS elements from 4 floats
__device__ __forceinline__ void store4(bf16 *p, float a, float b, float c, float d) {
    bf16x4 x = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
    *reinterpret_cast<bf16x4 *>(p) = x;
}
__device__ __forceinline__ void store4(float *p, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4 *>(p) = f32x4{a, b, c, d};
}

// ------------------------------------------------------- staging helpers
// A 16-byte global load holds VEC consecutive elements of one row.
__device__ __forceinline__ void stage_row(bf16 *dst, const uint4 &raw) {  // 8 bf16, 8-byte aligned
    uint2 *d = reinterpret_cast<uint2 *>(dst);
    d[0] = make_uint2(raw.x, raw.y);
    d[1] = make_uint2(raw.z, raw.w);
}
__device__ __forceinline__ void stage_row(float *dst, const uint4 &raw) {  // 4 floats, 16-byte aligned
    *reinterpret_cast<uint4 *>(dst) = raw;
}
// Transposed write of a 4-row x VEC-column block: column e of the block
// becomes 4 consecutive elements at dst + e * stride.
__device__ __forceinline__ void stage_transposed(bf16 *dst, int stride, const uint4 (&r)[4]) {
    const uint16_t *p0 = reinterpret_cast<const uint16_t *>(&r[0]);
    const uint16_t *p1 = reinterpret_cast<const uint16_t *>(&r[1]);
    const uint16_t *p2 = reinterpret_cast<const uint16_t *>(&r[2]);
    const uint16_t *p3 = reinterpret_cast<const uint16_t *>(&r[3]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint2 v = make_uint2((uint32_t)p0[e] | ((uint32_t)p1[e] << 16),
                             (uint32_t)p2[e] | ((uint32_t)p3[e] << 16));
        *reinterpret_cast<uint2 *>(dst + e * stride) = v;
    }
}
__device__ __forceinline__ void stage_transposed(float *dst, int stride, const uint4 (&r)[4]) {
    const uint32_t *p0 = reinterpret_cast<const uint32_t *>(&r[0]);
    const uint32_t *p1 = reinterpret_cast<const uint32_t *>(&r[1]);
    const uint32_t *p2 = reinterpret_cast<const uint32_t *>(&r[2]);
    const uint32_t *p3 = reinterpret_cast<const uint32_t *>(&r[3]);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        *reinterpret_cast<uint4 *>(dst + e * stride) = make_uint4(p0[e], p1[e], p2[e], p3[e]);
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// 4 consecutive I/O elements (one lane's slice of an output tile row)
template <typename IO> struct Vec4;
template <> struct Vec4<bf16> {
    typedef uint2 raw;
    static __device__ __forceinline__ raw load(const bf16 *p) { return *reinterpret_cast<const uint2 *>(p); }
    static __device__ __forceinline__ float get(const raw &r, int e) {
        const uint32_t w = e < 2 ? r.x : r.y;
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
    static __device__ __forceinline__ void store(bf16 *p, float a, float b, float c, float d) {
        bf16x4 x = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
        *reinterpret_cast<bf16x4 *>(p) = x;
    }
};
template <> struct Vec4<float> {
    typedef float4 raw;
    static __device__ __forceinline__ raw load(const float *p) { return *reinterpret_cast<const float4 *>(p); }
    static __device__ __forceinline__ float get(const raw &r, int e) {
        return e == 0 ? r.x : e == 1 ? r.y : e == 2 ? r.z : r.w;
    }
    static __device__ __forceinline__ void store(float *p, float a, float b, float c, float d) {
        *reinterpret_cast<float4 *>(p) = make_float4(a, b, c, d);
    }
};

// ------------------------------------------------------------------ kernel
// STATE_ONLY: produce each segment's local state from a zero start (no
// outputs); the first pass of the segmented schedule.
template <typename IO, int L, int DKP, int BV, int NW, bool STATE_ONLY>
__global__ __launch_bounds__(64 * NW, 1) void mlstm_chunk_kernel(FwdArgs a) {
    using Cfg = PrefillCfg<IO, L, DKP, BV, NW>;
    using TS = typename Cfg::TS;
    constexpr bool SPLIT = Cfg::SPLIT;
    constexpr int NTH = Cfg::NTH, LP = Cfg::LP, NT = Cfg::NT, NCT = Cfg::NCT, MYT = Cfg::MYT;
    constexpr int NAT = Cfg::NAT, NKS = Cfg::NKS, NJS = Cfg::NJS, WC = Cfg::WC, NBT = Cfg::NBT;
    constexpr int QST = Cfg::QST, TST = Cfg::TST, VEC = Cfg::VEC, UQK = Cfg::UQK, UV = Cfg::UV;
    typedef Frag<SPLIT> F;

    __shared__ __attribute__((aligned(16))) TS Qs[L * QST];
    __shared__ __attribute__((aligned(16))) TS Ks[L * QST];
    __shared__ __attribute__((aligned(16))) TS KTs[DKP * TST];
    __shared__ __attribute__((aligned(16))) TS VTs[BV * TST];
    __shared__ __attribute__((aligned(16))) TS Ps[L * TST];
    __shared__ __attribute__((aligned(16))) float g_w[LP];
    __shared__ float g_u[LP], g_r[LP], g_s[LP], g_fl[LP];
    __shared__ float den_part[NCT * 16];
    __shared__ float qn[L];
    __shared__ float nst[DKP];
    __shared__ float sc[4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;

    // workgroup -> (pair, segment, column tile).  Hardware hands consecutive
    // workgroups to the 8 XCDs round robin; the remap gives each XCD a
    // contiguous range, so the column tiles of one pair (which read the same
    // Q and K) share an L2.
    const int nwg = gridDim.x;
    int logical = blockIdx.x;
    if ((nwg & 7) == 0) logical = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
    const int gseg = STATE_ONLY ? a.nseg - 1 : a.nseg;
    const int tile = logical % a.ntile;
    const int rest = logical / a.ntile;
    const int seg = rest % gseg;
    const int bh = rest / gseg;

    const int dk = a.dk, dv = a.dv, T = a.T;
    const int t_begin = seg * a.seg_len;
    const int t_end = min(t_begin + a.seg_len, T);
    const int nchunks = (t_end - t_begin + L - 1) / L;
    const int col0 = tile * BV;            // first value column of the workgroup
    const int wcol0 = wave * WC;           // first column of this wavefront (tile-local)
    const int bv_here = min(BV, dv - col0);

    const IO *qg = static_cast<const IO *>(a.q) + (size_t)bh * T * dk;
    const IO *kg = static_cast<const IO *>(a.k) + (size_t)bh * T * dk;
    const IO *vg = static_cast<const IO *>(a.v) + (size_t)bh * T * dv;
    const IO *og = static_cast<const IO *>(a.o) + (size_t)bh * T * dv;
    IO *hg = static_cast<IO *>(a.h) + (size_t)bh * T * dv;
    const float *igg = a.ig + (size_t)bh * T;
    const float *fgg = a.fg + (size_t)bh * T;

    // ---- zero the LDS tiles once: padding rows/columns and the upper
    // (never written) tiles of P must read as zero
    for (int e = tid; e < L * QST; e += NTH) { Qs[e] = (TS)0.0f; Ks[e] = (TS)0.0f; }
    for (int e = tid; e < DKP * TST; e += NTH) KTs[e] = (TS)0.0f;
    for (int e = tid; e < BV * TST; e += NTH) VTs[e] = (TS)0.0f;
    for (int e = tid; e < L * TST; e += NTH) Ps[e] = (TS)0.0f;
    for (int e = tid; e < LP; e += NTH) g_w[e] = 0.0f;

    // ---- initial state
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
    f32x4 Cr[NAT][NBT];
#pragma unroll
    for (int at = 0; at < NAT; ++at)
#pragma unroll
        for (int bt = 0; bt < NBT; ++bt) {
            const int b = col0 + wcol0 + 16 * bt + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * at + 4 * g4 + r;
                Cr[at][bt][r] = (Cs && row < dk && b < dv) ? Cs[(size_t)row * dv + b] : 0.0f;
            }
        }
    for (int e = tid; e < DKP; e += NTH) nst[e] = (ns && e < dk) ? ns[e] : 0.0f;

    // ---- staging: registers <- global (chunk c), LDS <- registers
    const int nvq = dk / VEC;                 // 16-byte vectors per Q/K row
    const int nvv = bv_here / VEC;            // 16-byte vectors per V row of this tile
    const int uqk = (L / 4) * nvq;
    const int uv = (L / 4) * nvv;
    uint4 rq[UQK][4], rk[UQK][4], rv[UV][4];
    // wavefront 0: the chunk's gates, token 64 h + lane in slot h
    constexpr int NGH = (L + 63) / 64;
    float gf[NGH], gi[NGH];
#pragma unroll
    for (int hh = 0; hh < NGH; ++hh) {
        gf[hh] = 0.0f;
        gi[hh] = -INFINITY;
    }

    auto load_chunk = [&](int c) {
        const int tc = t_begin + c * L;
#pragma unroll
        for (int u = 0; u < UQK; ++u) {
            const int idx = tid + u * NTH;
            const int quad = idx / max(nvq, 1), vec = idx - quad * nvq;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = tc + 4 * quad + r;
                const bool ok = idx < uqk && t < t_end;
                const size_t off = (size_t)t * dk + vec * VEC;
                if (!STATE_ONLY) rq[u][r] = ok ? *reinterpret_cast<const uint4 *>(qg + off) : zero4();
                rk[u][r] = ok ? *reinterpret_cast<const uint4 *>(kg + off) : zero4();
            }
        }
#pragma unroll
        for (int u = 0; u < UV; ++u) {
            const int idx = tid + u * NTH;
            const int quad = idx / max(nvv, 1), vec = idx - quad * nvv;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = tc + 4 * quad + r;
                const bool ok = idx < uv && t < t_end;
                rv[u][r] = ok ? *reinterpret_cast<const uint4 *>(vg + (size_t)t * dv + col0 + vec * VEC)
                              : zero4();
            }
        }
        if (wave == 0) {
#pragma unroll
            for (int hh = 0; hh < NGH; ++hh) {
                const int tok = 64 * hh + lane, t = tc + tok;
                const bool ok = tok < L && t < t_end;
                gf[hh] = ok ? fgg[t] : 0.0f;
                gi[hh] = ok ? igg[t] : -INFINITY;
            }
        }
    };
    auto write_chunk = [&]() {
#pragma unroll
        for (int u = 0; u < UQK; ++u) {
            const int idx = tid + u * NTH;
            if (idx < uqk) {
                const int quad = idx / nvq, vec = idx - quad * nvq;
                const int a0 = vec * VEC;
                if (!STATE_ONLY) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        stage_row(&Qs[(4 * quad + r) * QST + a0], rq[u][r]);
                        stage_row(&Ks[(4 * quad + r) * QST + a0], rk[u][r]);
                    }
                }
                stage_transposed(&KTs[a0 * TST + 4 * quad], TST, rk[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < UV; ++u) {
            const int idx = tid + u * NTH;
            if (idx < uv) {
                const int quad = idx / nvv, vec = idx - quad * nvv;
                stage_transposed(&VTs[(vec * VEC) * TST + 4 * quad], TST, rv[u]);
            }
        }
    };
    // wavefront 0: gate quantities of the staged chunk, one token per lane in
    // each 64-token part: the inclusive sums of f~ and the prefix maxima of
    // u run across the parts through the carries of the previous part's last
    // lane (tokens past the chunk or T have f~ = 0, i~ = -inf and leave both
    // unchanged)
    auto gate_prep = [&](float m_before) {
        float bcarry = 0.0f, pmcarry = -INFINITY, r_last = 0.0f, b_last = 0.0f;
        float uh[NGH];
#pragma unroll
        for (int hh = 0; hh < NGH; ++hh) {
            float b = gf[hh];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(b, off, 64);
                if (lane >= off) b += y;
            }
            b += bcarry;
            const float u = gi[hh] - b;
            float pm = u;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(pm, off, 64);
                if (lane >= off) pm = fmaxf(pm, y);
            }
            pm = fmaxf(pm, pmcarry);
            const float r = fmaxf(m_before, pm);
            const int tok = 64 * hh + lane;
            if (tok < L) {
                g_u[tok] = u;
                g_r[tok] = r;
                g_s[tok] = exp_e(m_before - r);
                g_fl[tok] = exp_e(-(b + r));
            }
            uh[hh] = u;
            if (hh == (L - 1) / 64) {  // the part holding the chunk's last token
                r_last = __shfl(r, (L - 1) % 64, 64);
                b_last = __shfl(b, (L - 1) % 64, 64);
            }
            bcarry = __shfl(b, 63, 64);
            pmcarry = __shfl(pm, 63, 64);
        }
#pragma unroll
        for (int hh = 0; hh < NGH; ++hh) {
            const int tok = 64 * hh + lane;
            if (tok < L) g_w[tok] = exp_e(uh[hh] - r_last);
        }
        if (lane == 0) {
            sc[0] = b_last + r_last;          // stabilizer after the chunk
            sc[1] = exp_e(m_before - r_last); // decay of the carried state
            sc[2] = b_last;                   // sum of the chunk's log forget gates
        }
    };

    // causal tiles (jt <= it) of S owned by this wavefront: t = wave + NW*x
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

    float g_total = 0.0f;  // sum of log forget gates over the segment

    if (nchunks > 0) {
        load_chunk(0);
        __syncthreads();  // LDS zeroing done
        write_chunk();
        if (wave == 0) gate_prep(m_prev);
    }
    __syncthreads();

    for (int c = 0; c < nchunks; ++c) {
        const int tc = t_begin + c * L;
        const float m_next = sc[0], s_last = sc[1];
        g_total += sc[2];
        if (c + 1 < nchunks) load_chunk(c + 1);

        if (!STATE_ONLY) {
            // output-gate inputs of this chunk for this lane's output slots
            typename Vec4<IO>::raw orw[NT][NBT];
#pragma unroll
            for (int it = 0; it < NT; ++it)
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt) {
                    const int t = tc + 16 * it + l16;
                    const int b = col0 + wcol0 + 16 * bt + 4 * g4;
                    if (t < t_end && b < dv) orw[it][bt] = Vec4<IO>::load(og + (size_t)t * dv + b);
                }

            // q_i . n' for every token of the chunk (n' of the previous state)
            {
                constexpr int TPRQ = NTH / L;
                constexpr int SPAN = DKP / TPRQ;
                const int i = tid / TPRQ, p = tid % TPRQ;
                float acc = 0.0f;
#pragma unroll 8
                for (int e = 0; e < SPAN; ++e) acc += to_f(Qs[i * QST + p * SPAN + e]) * nst[p * SPAN + e];
#pragma unroll
                for (int off = 1; off < TPRQ; off <<= 1) acc += __shfl_xor(acc, off, 64);
                if (p == 0) qn[i] = acc;
            }

            // O^T = C'^T Q^T and the causal tiles of S^T = K Q^T, over d_qk
            f32x4 Ot[NBT][NT];
            f32x4 St[MYT];
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt)
#pragma unroll
                for (int it = 0; it < NT; ++it) Ot[bt][it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int x = 0; x < MYT; ++x) St[x] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                // C' in parts for either I/O dtype (three against float32 q,
                // high part and remainder against bf16 q): a read-out through
                // C' rounded to bf16 alone loses tokens whose C'^T q cancels
                typename std::conditional<SPLIT, Frag<true>, Frag2>::type ac[NBT];
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt) {
                    const float x[8] = {Cr[2 * ks][bt][0], Cr[2 * ks][bt][1], Cr[2 * ks][bt][2],
                                        Cr[2 * ks][bt][3], Cr[2 * ks + 1][bt][0], Cr[2 * ks + 1][bt][1],
                                        Cr[2 * ks + 1][bt][2], Cr[2 * ks + 1][bt][3]};
                    set_frag(ac[bt], x);
                }
#pragma unroll
                for (int it = 0; it < NT; ++it) {
                    F bq;
                    load_frag_perm(bq, &Qs[(16 * it + l16) * QST + 32 * ks + 4 * g4]);
#pragma unroll
                    for (int bt = 0; bt < NBT; ++bt) Ot[bt][it] = mma(ac[bt], bq, Ot[bt][it]);
#pragma unroll
                    for (int x = 0; x < MYT; ++x) {
                        if (tok[x] && tit[x] == it) {
                            F ak;
                            load_frag_perm(ak, &Ks[(16 * tjt[x] + l16) * QST + 32 * ks + 4 * g4]);
                            St[x] = mma(ak, bq, St[x]);
                        }
                    }
                }
            }

            // P = S (x) e^{u_j - r_i} (causal) -> LDS; column sums -> den_part
#pragma unroll
            for (int x = 0; x < MYT; ++x) {
                if (tok[x]) {
                    const int i = 16 * tit[x] + l16;
                    const float ri = g_r[i];
                    float p[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 16 * tjt[x] + 4 * g4 + r;
                        p[r] = (j <= i) ? St[x][r] * exp_e(g_u[j] - ri) : 0.0f;
                    }
                    store4(&Ps[i * TST + 16 * tjt[x] + 4 * g4], p[0], p[1], p[2], p[3]);
                    float cs = (p[0] + p[1]) + (p[2] + p[3]);
                    cs += __shfl_xor(cs, 16, 64);
                    cs += __shfl_xor(cs, 32, 64);
                    if (g4 == 0) den_part[(wave + NW * x) * 16 + l16] = cs;
                }
            }
            // inter-chunk part weighted by e^{m - r_i}
#pragma unroll
            for (int it = 0; it < NT; ++it) {
                const float si = g_s[16 * it + l16];
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt) Ot[bt][it] *= si;
            }
            __syncthreads();  // P, den_part, qn visible

            // O^T += V^T P^T (P is zero above the diagonal: skip those k-steps)
#pragma unroll
            for (int js = 0; js < NJS; ++js) {
                F av[NBT];
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt)
                    load_frag_nat(av[bt], &VTs[(wcol0 + 16 * bt + l16) * TST + 32 * js + 8 * g4]);
#pragma unroll
                for (int it = 0; it < NT; ++it) {
                    if (32 * js <= 16 * it + 15) {
                        F bp;
                        load_frag_nat(bp, &Ps[(16 * it + l16) * TST + 32 * js + 8 * g4]);
#pragma unroll
                        for (int bt = 0; bt < NBT; ++bt) Ot[bt][it] = mma(av[bt], bp, Ot[bt][it]);
                    }
                }
            }

            // h = sigmoid(o~) * num / max(|den|, e^{-M})
#pragma unroll
            for (int it = 0; it < NT; ++it) {
                const int i = 16 * it + l16;
                const int t = tc + i;
                float den = g_s[i] * qn[i];
#pragma unroll
                for (int jt = 0; jt <= it; ++jt) den += den_part[(it * (it + 1) / 2 + jt) * 16 + l16];
                const float inv = 1.0f / fmaxf(fabsf(den), g_fl[i]);
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt) {
                    const int b = col0 + wcol0 + 16 * bt + 4 * g4;
                    if (t < t_end && b < dv) {
                        const typename Vec4<IO>::raw &o4 = orw[it][bt];
                        Vec4<IO>::store(hg + (size_t)t * dv + b,
                                        sigmoid(Vec4<IO>::get(o4, 0)) * Ot[bt][it][0] * inv,
                                        sigmoid(Vec4<IO>::get(o4, 1)) * Ot[bt][it][1] * inv,
                                        sigmoid(Vec4<IO>::get(o4, 2)) * Ot[bt][it][2] * inv,
                                        sigmoid(Vec4<IO>::get(o4, 3)) * Ot[bt][it][3] * inv);
                    }
                }
            }
        }

        // C' <- e^{m - r_last} C' + K^T (w (x) V)
#pragma unroll
        for (int at = 0; at < NAT; ++at)
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt) Cr[at][bt] *= s_last;
#pragma unroll
        for (int js = 0; js < NJS; ++js) {
            float w8[8];
            {
                const f32x4 w0 = *reinterpret_cast<const f32x4 *>(&g_w[32 * js + 8 * g4]);
                const f32x4 w1 = *reinterpret_cast<const f32x4 *>(&g_w[32 * js + 8 * g4 + 4]);
                w8[0] = w0[0]; w8[1] = w0[1]; w8[2] = w0[2]; w8[3] = w0[3];
                w8[4] = w1[0]; w8[5] = w1[1]; w8[6] = w1[2]; w8[7] = w1[3];
            }
            F bw[NBT];
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt)
                load_frag_nat_scaled(bw[bt], &VTs[(wcol0 + 16 * bt + l16) * TST + 32 * js + 8 * g4], w8);
#pragma unroll
            for (int at = 0; at < NAT; ++at) {
                F ak;
                load_frag_nat(ak, &KTs[(16 * at + l16) * TST + 32 * js + 8 * g4]);
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt) Cr[at][bt] = mma(ak, bw[bt], Cr[at][bt]);
            }
        }
        // n' <- e^{m - r_last} n' + K^T w
        for (int e = tid; e < DKP; e += NTH) {
            float acc = 0.0f;
#pragma unroll 8
            for (int j = 0; j < L; ++j) acc += g_w[j] * to_f(KTs[e * TST + j]);
            nst[e] = s_last * nst[e] + acc;
        }
        m_prev = m_next;
        __syncthreads();  // all reads of this chunk's tiles are done

        if (c + 1 < nchunks) {
            write_chunk();
            if (wave == 0) gate_prep(m_prev);
        }
        __syncthreads();
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
        for (int at = 0; at < NAT; ++at)
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt) {
                const int b = col0 + wcol0 + 16 * bt + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * at + 4 * g4 + r;
                    if (row < dk && b < dv) Cdst[(size_t)row * dv + b] = Cr[at][bt][r];
                }
            }
        if (tile == 0) {
            for (int e = tid; e < dk; e += NTH) ndst[e] = nst[e];
            if (tid == 0) mdst[0] = m_prev;
        }
    }
}

}  // namespace mlstm
