// kda_chunked.hip -- chunkwise KDA forward for gfx950 (MI355X).
//
// The pages name a chunkwise algorithm built on the Diagonal-Plus-Low-Rank
// state transition (akshathtiwari.co.in "Kimi Delta Attention" explainer) that
// regroups the recurrence into matrix products (daily.dev summary of "You
// Could Have Come Up with Kimi Delta Attention"); they do not print it, so
// the form below is derived from the recurrence
//     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t.
//
// Per chunk of C = 64 tokens with entry state S (d_k x d_v), Gamma_r the
// inclusive cumulative log-decay per key channel inside the chunk:
//   A      = strict_lower(Diag(beta) K_up K_dn^T)      A_ri = beta_r sum_c k_rc k_ic e^{Gamma_rc - Gamma_ic}
//   T'     = (I + A)^{-1} Diag(beta)
//   U      = T' (V - K_up S)                             K_up = K * e^{Gamma}
//   O      = Q_up S + tril_incl(Q_up K_dn^T) U           Q_up = Q * e^{Gamma}
//   S_next = Diag(e^{Gamma_last}) S + K_right^T U        K_right = K * e^{Gamma_last - Gamma}
//
// Work split: one 256-thread workgroup (4 waves) owns one (sequence, head,
// value-slice) and walks that sequence's chunks in order.  The fp32 state
// slice lives in MFMA accumulator registers for the whole sequence: each wave
// owns 16-column strips of S.  The rows of every accumulator tile are
// assigned so that an accumulator can be fed straight back as the B operand
// of the next MFMA in natural k order (see rowmap), so S, V - K_up S and U
// never round-trip through LDS.
//
// Per chunk (all waves):
//   A1  wave R loads rows 16R..16R+15 of g, scans the log-decay along rows
//       (DPP), forms lambda = Gamma - Gamma_mid(R) relative to the middle of
//       its 16-row block, and publishes block sums.
//   A2  one thread per key channel turns block sums into the few per-chunk
//       factors (block-to-block decays, e^{Gamma_last}).
//   A3  wave R scales its k / q rows: k a, q a, k b with a = e^{lambda},
//       b = e^{-lambda}; K_up, Q_up, K_right^T go to LDS.
//   A4  wave R forms its row block of A and of the intra-chunk output matrix
//       P on MFMA: diagonal tile from registers, off-diagonal tiles against
//       k b (from LDS) times the block-to-block decay.
//   A5  T = (I + A)^{-1}: 16x16 diagonal blocks by forward substitution,
//       off-diagonal blocks by fp32 MFMA, then T' = T Diag(beta).
//   B   per 16-column strip: Y = K_up S, O1 = Q_up S, U = T'(V - Y),
//       O = O1 + P U, S = Diag(gamma) S + K_right^T U.
//
// Exponent range.  All decay factors of the form e^{Gamma_r - Gamma_i} with
// r >= i are <= 1.  Splitting them at a reference row inside a 16-row block
// gives one factor above 1; the fast path is taken when every |lambda| in
// the chunk is <= 96 in log2 units (no factor leaves [2^-96, 2^96]).  A chunk
// with stronger decay inside a 16-row block takes an exact slower path that
// forms A and P entry by entry with e^{Gamma_r - Gamma_i} evaluated directly.
#include <mutex>

#include "kda_device.h"

namespace kda {

constexpr int CH = 64;   // chunk length (tokens)

struct ChunkParams {
    const void *q, *k, *v, *g, *beta;
    const float *S0;
    float *S_T;
    void *o;
    const int32_t *cu_seqlens;   // NULL -> dense
    const int32_t *order;        // sequence processing order (NULL -> identity)
    const int32_t *state_idx;    // slot map of S0 / S_T rows (NULL -> row = sequence)
    int pool;       // rows of S0 / S_T when state_idx is set
    int gate;       // GATE_CHANNEL / GATE_HEAD / GATE_NONE
    int prep;       // PREP_L2NORM | PREP_SOFTPLUS
    int T;          // tokens per batch row (dense)
    int H;
    int DV;         // full value dimension
    int units;      // num_seqs * H
    int nslices;    // DV / DVS
};

// Per-mode operand conventions.  RUN consecutive key channels form one
// lane's share of one MFMA k-step group:
//   bf16: v_mfma_f32_16x16x32_bf16, lane (row m, group j) supplies k = 8j..8j+7
//   f32 : v_mfma_f32_16x16x4f32, four steps; step i, lane group j <-> k = 4j + i
// A "run" rho covers logical k in [4*RUN*rho, 4*RUN*rho + 4*RUN); lane group
// j owns logical k = 4*RUN*rho + RUN*j + (0..RUN-1).
template <bool F32> struct Mode;
template <> struct Mode<false> {
    using in_t = bf16_t;
    using op_t = bf16_t;
    using frag_t = bf16x8;
    static constexpr int RUN = 8;
    static constexpr int PAD = 8;   // elements: 16 bytes
};
template <> struct Mode<true> {
    using in_t = float;
    using op_t = float;
    using frag_t = f32x4;
    static constexpr int RUN = 4;
    static constexpr int PAD = 4;
};

// Row (logical index) held by accumulator tile (run rho, half h) at tile row m.
// With it, the 4 registers of a lane of two (bf16) or one (f32) accumulator
// tiles are exactly the lane's B-operand k-slots of run rho in natural order.
template <int RUN>
__device__ __forceinline__ int rowmap(int rho, int h, int m) {
    return 4 * RUN * rho + RUN * (m >> 2) + 4 * h + (m & 3);
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <bool F32>
__device__ __forceinline__ f32x4 mma_run(f32x4 acc, typename Mode<F32>::frag_t a,
                                         typename Mode<F32>::frag_t b) {
    if constexpr (F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = mfma_f32(a[i], b[i], acc);
        return acc;
    } else {
        return mfma_bf16(a, b, acc);
    }
}

// B-operand fragment of run rho from accumulator tiles (rowmap layout).
template <bool F32>
__device__ __forceinline__ typename Mode<F32>::frag_t acc_frag(const f32x4 *tiles, int rho) {
    if constexpr (F32) {
        return tiles[rho];
    } else {
        const f32x4 lo = tiles[2 * rho], hi = tiles[2 * rho + 1];
        bf16x8 f;
        f[0] = (__bf16)lo[0]; f[1] = (__bf16)lo[1]; f[2] = (__bf16)lo[2]; f[3] = (__bf16)lo[3];
        f[4] = (__bf16)hi[0]; f[5] = (__bf16)hi[1]; f[6] = (__bf16)hi[2]; f[7] = (__bf16)hi[3];
        return f;
    }
}

template <bool F32>
__device__ __forceinline__ typename Mode<F32>::frag_t to_frag(const float *x) {
    typename Mode<F32>::frag_t f;
    if constexpr (F32) {
        f[0] = x[0]; f[1] = x[1]; f[2] = x[2]; f[3] = x[3];
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (__bf16)x[e];
    }
    return f;
}

// Store RUN fp32 values as operands (16 bytes either way).
template <bool F32>
__device__ __forceinline__ void store_run(typename Mode<F32>::op_t *dst, const float *x) {
    *reinterpret_cast<typename Mode<F32>::frag_t *>(dst) = to_frag<F32>(x);
}

// Convert 16 raw bytes of inputs (8 bf16 or 4 fp32) to fp32.
template <bool F32>
__device__ __forceinline__ void raw_to_f32(const uint4 t, float *x) {
    if constexpr (F32) {
        x[0] = __uint_as_float(t.x); x[1] = __uint_as_float(t.y);
        x[2] = __uint_as_float(t.z); x[3] = __uint_as_float(t.w);
    } else {
        const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = __uint_as_float(w[e] << 16);
            x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    }
}

__device__ __forceinline__ float dpp_row_shr(float x, int n) {
    // lanes m < n of each 16-lane row receive 0
    switch (n) {
    case 1: return __builtin_amdgcn_update_dpp(0.0f, x, 0x111, 0xf, 0xf, false);
    case 2: return __builtin_amdgcn_update_dpp(0.0f, x, 0x112, 0xf, 0xf, false);
    case 4: return __builtin_amdgcn_update_dpp(0.0f, x, 0x114, 0xf, 0xf, false);
    default: return __builtin_amdgcn_update_dpp(0.0f, x, 0x118, 0xf, 0xf, false);
    }
}
__device__ __forceinline__ float dpp_row_share8(float x) {
    return __builtin_amdgcn_update_dpp(0.0f, x, 0x158, 0xf, 0xf, false);
}

// LDS layout (bytes), per instantiation.
template <int DK, bool F32>
struct Lds {
    using op_t = typename Mode<F32>::op_t;
    static constexpr int PAD = Mode<F32>::PAD;
    static constexpr int LDK = DK + PAD;          // row stride of [64][DK] operand arrays
    static constexpr int LCH = CH + PAD;          // row stride of [*][64] operand arrays
    static constexpr int LF = CH + 4;             // row stride of fp32 [64][64] arrays
    // fp32 operands leave no room for separate K_right^T, T and T' arrays at
    // d_k = 128 (217 KB), so the fp32 layout drops all three: K_right is read
    // from the k b rows times a per-block channel factor, T is built inside A's
    // array (diagonal blocks in place, block (R, I) at the mirror position
    // (I, R), which A never uses), and T' then overwrites A's lower blocks.
    static constexpr int KU = 0;                                         // K_up  [64][LDK]
    static constexpr int QU = KU + CH * LDK * (int)sizeof(op_t);         // Q_up  [64][LDK]
    static constexpr int KB = QU + CH * LDK * (int)sizeof(op_t);         // k b   [64][LDK]
    static constexpr int KRT = KB + CH * LDK * (int)sizeof(op_t);        // K_right^T [DK][LCH] (bf16)
    static constexpr int AM = F32 ? KRT : KRT + DK * LCH * (int)sizeof(op_t);   // A fp32 [64][LF]
    static constexpr int TF = F32 ? AM : AM + CH * LF * 4;               // T fp32 [64][LF]
    static constexpr int TP = F32 ? AM : TF + CH * LF * 4;               // T' op [64][LCH]
    static constexpr int PM = F32 ? AM + CH * LF * 4 : TP + CH * LCH * (int)sizeof(op_t);   // P op [64][LCH]
    static constexpr int FAC = PM + CH * LCH * (int)sizeof(op_t);        // factors fp32 [20][DK]
    static constexpr int TOT = FAC + 20 * DK * 4;                        // block sums [4][2][DK] + dummy
    static constexpr int BETA = TOT + (8 * DK + 256 + DK) * 4;          // beta [64]
    static constexpr int BYTES = BETA + CH * 4;
    // slow path: Gamma fp32 [64][DK] over k b (fp32) or over A..T (bf16)
    static constexpr int GAM = F32 ? KB : AM;
    static_assert(!F32 || (LCH == LF && CH * DK * 4 <= CH * LDK * 4), "fp32 aliasing");
    static_assert(F32 || CH * DK * 4 <= 2 * CH * LF * 4, "slow-path Gamma fits");
    static_assert(BYTES <= 160 * 1024, "LDS");
};
// Position of element (r, c) of block (Rb, Ib), Ib <= Rb, of T in the fp32
// layout: diagonal blocks in place, the others at the mirror block (Ib, Rb).
template <int LF>
__device__ __forceinline__ int t_at(int Rb, int Ib, int r, int c) {
    return Rb == Ib ? (16 * Rb + r) * LF + 16 * Ib + c : (16 * Ib + r) * LF + 16 * Rb + c;
}
// factor rows in Lds::FAC
constexpr int F_B = 0;      // e^{Gamma_mid(R)}, R = 0..3
constexpr int F_W = 4;      // e^{Gamma_mid(R) - Gamma_mid(I)}, (1,0),(2,0),(2,1),(3,0),(3,1),(3,2)
constexpr int F_GAM = 10;   // e^{Gamma_last}
constexpr int F_Z = 11;     // e^{Gamma_last - Gamma_mid(R)}, R = 0..3
constexpr int F_P = 15;     // Gamma at the end of block R-1 (log2), R = 0..3; 19: Gamma_last (log2)
__device__ __forceinline__ int w_index(int R, int I) { return F_W + (R * (R - 1)) / 2 + I; }

template <int DK, int NSTRIP, bool F32>
__global__ __launch_bounds__(256, 1) void chunked_fwd_kernel(ChunkParams p)
{
    using M = Mode<F32>;
    using in_t = typename M::in_t;
    using op_t = typename M::op_t;
    using frag_t = typename M::frag_t;
    using L = Lds<DK, F32>;
    constexpr int RUN = M::RUN;
    constexpr int NCH = DK / 4;          // key channels per lane in the prep phase
    constexpr int NRUN = NCH / RUN;      // runs over d_k
    constexpr int TPR = RUN / 4;         // accumulator tiles per run (2 bf16, 1 f32)
    constexpr int NKT = DK / 16;         // accumulator tiles over d_k (state rows)
    constexpr int DVS = 64 * NSTRIP;     // value columns per workgroup

    __shared__ __attribute__((aligned(16))) unsigned char smem[L::BYTES];
    op_t *sKU = reinterpret_cast<op_t *>(smem + L::KU);
    op_t *sQU = reinterpret_cast<op_t *>(smem + L::QU);
    op_t *sKRt = reinterpret_cast<op_t *>(smem + L::KRT);
    op_t *sKB = reinterpret_cast<op_t *>(smem + L::KB);
    float *sA = reinterpret_cast<float *>(smem + L::AM);
    float *sTf = reinterpret_cast<float *>(smem + L::TF);
    op_t *sTp = reinterpret_cast<op_t *>(smem + L::TP);
    op_t *sP = reinterpret_cast<op_t *>(smem + L::PM);
    float *sFac = reinterpret_cast<float *>(smem + L::FAC);
    float *sTot = reinterpret_cast<float *>(smem + L::TOT);
    float *sBeta = reinterpret_cast<float *>(smem + L::BETA);
    float *sGam = reinterpret_cast<float *>(smem + L::GAM);  // slow path only

    // ---- work unit: XCD-aware (sequence, head, slice) ------------------------
    // Blocks b and b + 8 run on the same XCD (round-robin dispatch), so the
    // slices of one (sequence, head) are given ids 8 apart and share that
    // XCD's L2 for their common k / q / g reads.
    const int NS = p.nslices;
    const int bid = blockIdx.x;
    const int grp = bid / (8 * NS);
    const int xcd = bid & 7;
    const int slice = (bid >> 3) % NS;
    const int sh = grp * 8 + xcd;
    if (sh >= p.units) return;
    const int H = p.H, DV = p.DV;
    const int seq_rank = sh / H, head = sh - (sh / H) * H;
    const int seq = p.order ? p.order[seq_rank] : seq_rank;
    const long strow = state_row(p.state_idx, p.pool, seq);
    long t0, len;
    if (p.cu_seqlens) {
        t0 = p.cu_seqlens[seq];
        len = (long)p.cu_seqlens[seq + 1] - t0;
    } else {
        t0 = (long)seq * p.T;
        len = p.T;
    }
    const int col0 = slice * DVS;

    const int tid = threadIdx.x;
    // the wave index is uniform across a wave; say so, so that everything
    // derived from it (chunk ids, row bounds) lives in scalar registers
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, jg = lane >> 4, mr = lane & 15;

    const in_t *gq = static_cast<const in_t *>(p.q);
    const in_t *gk = static_cast<const in_t *>(p.k);
    const in_t *gv = static_cast<const in_t *>(p.v);
    const in_t *gg = static_cast<const in_t *>(p.g);
    const in_t *gb = static_cast<const in_t *>(p.beta);
    in_t *go = static_cast<in_t *>(p.o);

    // Upper blocks of T' and P stay zero for the whole sequence.
    for (int idx = tid; idx < CH * CH; idx += 256) {
        const int r = idx / CH, c = idx % CH;
        if ((c >> 4) > (r >> 4)) {
            store_elem(&sTp[r * L::LCH + c], 0.0f);
            store_elem(&sP[r * L::LCH + c], 0.0f);
        }
    }

    const int R = w;                  // prep row block of this wave
    const int rloc = 16 * R + mr;     // prep row (token within chunk) of this lane
    const uint32_t tokstride_k = (uint32_t)H * DK;   // elements between tokens (q, k, g)
    const uint32_t tokstride_v = (uint32_t)H * DV;   // elements between tokens (v, o)

    // ---- prefetch registers: raw bits of one chunk's inputs -----------------
    // g / k / q rows of this lane's prep row (RUN channels per run), beta of
    // that row, and v at the rows / columns this lane's accumulator tiles hold.
    // Rows past the chunk's end are read at the last valid row (always in
    // bounds) and masked where they are used, so no load sits behind a branch.
    uint4 rawg[NRUN], rawk[NRUN], rawq[NRUN];
    uint32_t rawb;
    uint32_t rawv[NSTRIP][16];

    auto load_prep = [&](long cs, int cl) {
        const uint32_t rr_ = (uint32_t)(rloc < cl ? rloc : cl - 1);
        const size_t tb = ((size_t)(t0 + cs) * H + head);
        const in_t *bg = gg + tb * DK, *bk = gk + tb * DK, *bq = gq + tb * DK;
        const uint32_t ro = rr_ * tokstride_k + RUN * jg;
        // a per-head gate is broadcast over the lane's channels (the scans
        // below then see equal values on every channel); no gate reads as 0
        uint32_t gbits = 0u;
        if (p.gate == GATE_HEAD) {
            if constexpr (F32) gbits = __float_as_uint(gg[tb + (size_t)rr_ * H]);
            else gbits = (uint32_t)gg[tb + (size_t)rr_ * H].x * 0x00010001u;
        }
#pragma unroll
        for (int rr = 0; rr < NRUN; ++rr) {
            if (p.gate == GATE_CHANNEL) rawg[rr] = *reinterpret_cast<const uint4 *>(bg + ro + 4 * RUN * rr);
            else rawg[rr] = make_uint4(gbits, gbits, gbits, gbits);
            rawk[rr] = *reinterpret_cast<const uint4 *>(bk + ro + 4 * RUN * rr);
            rawq[rr] = *reinterpret_cast<const uint4 *>(bq + ro + 4 * RUN * rr);
        }
        // kept raw: converting here would make the wait counter (in order)
        // drain every load issued before this one
        if constexpr (F32)
            rawb = __float_as_uint(gb[tb + (size_t)rr_ * H]);
        else
            rawb = (uint32_t)gb[tb + (size_t)rr_ * H].x;
    };
    auto load_v = [&](long cs, int cl) {
        const in_t *bv = gv + ((size_t)(t0 + cs) * H + head) * DV + col0;
#pragma unroll
        for (int s = 0; s < NSTRIP; ++s) {
            const uint32_t co = 16 * (w + 4 * s) + mr;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = rowmap<RUN>(tt / TPR, tt % TPR, 4 * jg + i);
                    const uint32_t crow = (uint32_t)(row < cl ? row : cl - 1);
                    if constexpr (F32)
                        rawv[s][4 * tt + i] = __float_as_uint(bv[crow * tokstride_v + co]);
                    else
                        rawv[s][4 * tt + i] = (uint32_t)bv[crow * tokstride_v + co].x;
                }
        }
    };
    if (len > 0) {
        const int cl0 = (int)(len < CH ? len : CH);
        load_prep(0, cl0);
        load_v(0, cl0);
    }

    // ---- state: NSTRIP strips x NKT tiles, rowmap rows, column = strip col + mr
    f32x4 S[NSTRIP][NKT];
    {
#pragma unroll
        for (int s = 0; s < NSTRIP; ++s)
#pragma unroll
            for (int tt = 0; tt < NKT; ++tt) S[s][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (p.S0 && strow >= 0) {
            const float *s0 = p.S0 + ((size_t)strow * H + head) * DK * DV + col0;
#pragma unroll
            for (int s = 0; s < NSTRIP; ++s) {
                const uint32_t co = 16 * (w + 4 * s) + mr;
#pragma unroll
                for (int tt = 0; tt < NKT; ++tt) {
                    const int rho = tt / TPR, h = tt % TPR;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t row = rowmap<RUN>(rho, h, 4 * jg + i);
                        S[s][tt][i] = s0[row * DV + co];
                    }
                }
            }
        }
    }

    for (long c0 = 0; c0 < len; c0 += CH) {
        const int clen = (int)((len - c0) < CH ? (len - c0) : CH);
        const bool rvalid = rloc < clen;
        // L2 normalisation of this lane's k and q row, whose channels are
        // spread over the four lanes 16 apart (factors 1 when not asked for)
        float ikn = 1.0f, iqn = 1.0f;
        if (p.prep & PREP_L2NORM) {
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int rr = 0; rr < NRUN; ++rr) {
                float kk[RUN], qq[RUN];
                raw_to_f32<F32>(rawk[rr], kk);
                raw_to_f32<F32>(rawq[rr], qq);
#pragma unroll
                for (int e = 0; e < RUN; ++e) {
                    sk += kk[e] * kk[e];
                    sq += qq[e] * qq[e];
                }
            }
            sk += __shfl_xor(sk, 16);
            sk += __shfl_xor(sk, 32);
            sq += __shfl_xor(sq, 16);
            sq += __shfl_xor(sq, 32);
            ikn = inv_norm(sk);
            iqn = inv_norm(sq);
        }
        auto load_kq = [&](int rr, float *kk, float *qq) {
            raw_to_f32<F32>(rawk[rr], kk);
            raw_to_f32<F32>(rawq[rr], qq);
#pragma unroll
            for (int e = 0; e < RUN; ++e) {
                kk[e] *= ikn;
                qq[e] *= iqn;
            }
        };
        const bool has_next = c0 + CH < len;
        const int clen_next = has_next ? (int)((len - c0 - CH) < CH ? (len - c0 - CH) : CH) : 0;

        // ================= A1: log-decay scan along rows =====================
        float lam[NCH];      // Gamma_r - Gamma_mid(R)   (log2)
        bool fast_ok = true;
        // rows 8 (block middle) and 15 (block end) publish their running sums;
        // every other lane writes to its own dummy slot, so there is no branch
        const int tot_base = (mr == 8) ? (2 * R + 0) * DK : (mr == 15) ? (2 * R + 1) * DK
                                                                         : 8 * DK + 64 * w + lane - RUN * jg;
#pragma unroll
        for (int rr = 0; rr < NRUN; ++rr) {
            const int cbase = 4 * RUN * rr + RUN * jg;
            float x[RUN];
            raw_to_f32<F32>(rawg[rr], x);
#pragma unroll
            for (int e = 0; e < RUN; ++e) {
                float v = !rvalid ? 0.0f
                        : (p.prep & PREP_SOFTPLUS) && p.gate != GATE_NONE ? log2_alpha_softplus(x[e])
                                                                          : x[e] * kLog2e;
                v += dpp_row_shr(v, 1);
                v += dpp_row_shr(v, 2);
                v += dpp_row_shr(v, 4);
                v += dpp_row_shr(v, 8);
                const float mid = dpp_row_share8(v);
                const float lm = v - mid;
                lam[rr * RUN + e] = lm;
                fast_ok = fast_ok && (fabsf(lm) <= 96.0f);
                sTot[tot_base + ((mr == 8 || mr == 15) ? cbase + e : RUN * jg)] = v;
            }
        }
        if (jg == 0) sBeta[rloc] = rvalid ? __uint_as_float(F32 ? rawb : rawb << 16) : 0.0f;
        const bool slow = __syncthreads_or(!fast_ok);

        // ================= A2: per-channel chunk factors ======================
        if (tid < DK) {
            const int c = tid;
            float Lm[4], Lt[4], Pb[4], Gm[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                Lm[b] = sTot[(2 * b + 0) * DK + c];
                Lt[b] = sTot[(2 * b + 1) * DK + c];
            }
            Pb[0] = 0.0f;
            Pb[1] = Lt[0];
            Pb[2] = Pb[1] + Lt[1];
            Pb[3] = Pb[2] + Lt[2];
            const float Glast = Pb[3] + Lt[3];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                Gm[b] = Pb[b] + Lm[b];
                // K_up is stored negated so that V + (-K_up) S accumulates directly
                sFac[(F_B + b) * DK + c] = -__builtin_amdgcn_exp2f(Gm[b]);
                sFac[(F_Z + b) * DK + c] = __builtin_amdgcn_exp2f(Glast - Gm[b]);
                sFac[(F_P + b) * DK + c] = Pb[b];
            }
#pragma unroll
            for (int b = 1; b < 4; ++b)
#pragma unroll
                for (int i = 0; i < b; ++i)
                    sFac[w_index(b, i) * DK + c] = __builtin_amdgcn_exp2f(Gm[b] - Gm[i]);
            sFac[F_GAM * DK + c] = __builtin_amdgcn_exp2f(Glast);
            sFac[(F_P + 4) * DK + c] = Glast;
        }
        __syncthreads();

        // ================= A3/A4: operands, A and P ==========================
        if (!slow) {
            frag_t fka[NRUN], fqa[NRUN], fkb[NRUN];
#pragma unroll
            for (int rr = 0; rr < NRUN; ++rr) {
                const int cbase = 4 * RUN * rr + RUN * jg;
                float kk[RUN], qq[RUN];
                load_kq(rr, kk, qq);
                float ka[RUN], qa[RUN], kb[RUN], ku[RUN], qu[RUN], kr[RUN];
#pragma unroll
                for (int e = 0; e < RUN; ++e) {
                    const int c = cbase + e;
                    const float lm = lam[rr * RUN + e];
                    const float kv = rvalid ? kk[e] : 0.0f, qv = rvalid ? qq[e] : 0.0f;
                    const float a = __builtin_amdgcn_exp2f(lm);
                    const float b = __builtin_amdgcn_exp2f(-lm);
                    ka[e] = kv * a;
                    qa[e] = qv * a;
                    kb[e] = kv * b;
                    const float Bf = sFac[(F_B + R) * DK + c];
                    ku[e] = ka[e] * Bf;
                    qu[e] = -qa[e] * Bf;
                    kr[e] = kb[e] * sFac[(F_Z + R) * DK + c];
                }
                fka[rr] = to_frag<F32>(ka);
                fqa[rr] = to_frag<F32>(qa);
                fkb[rr] = to_frag<F32>(kb);
                store_run<F32>(&sKU[rloc * L::LDK + cbase], ku);
                store_run<F32>(&sQU[rloc * L::LDK + cbase], qu);
                store_run<F32>(&sKB[rloc * L::LDK + cbase], kb);
                if constexpr (!F32) {
#pragma unroll
                    for (int e = 0; e < RUN; ++e) store_elem(&sKRt[(cbase + e) * L::LCH + rloc], kr[e]);
                }
            }
            // (at d_k = 128 the next chunk's rows are loaded after the A / P
            // tiles, whose operand registers would otherwise spill)
            if (DK <= 64 && has_next) load_prep(c0 + CH, clen_next);
            __syncthreads();

            // wave R: tiles (R, I), I = 0..R
            for (int I = 0; I <= R; ++I) {
                f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
                if (I == R) {
#pragma unroll
                    for (int rr = 0; rr < NRUN; ++rr) {
                        accA = mma_run<F32>(accA, fka[rr], fkb[rr]);
                        accP = mma_run<F32>(accP, fqa[rr], fkb[rr]);
                    }
                } else {
                    const int wrow = w_index(R, I);
#pragma unroll
                    for (int rr = 0; rr < NRUN; ++rr) {
                        const int cbase = 4 * RUN * rr + RUN * jg;
                        float cv[RUN];
                        const op_t *src = &sKB[(16 * I + mr) * L::LDK + cbase];
#pragma unroll
                        for (int e = 0; e < RUN; ++e)
                            cv[e] = load_elem(src + e) * sFac[wrow * DK + cbase + e];
                        const frag_t fc = to_frag<F32>(cv);
                        accA = mma_run<F32>(accA, fka[rr], fc);
                        accP = mma_run<F32>(accP, fqa[rr], fc);
                    }
                }
                // C layout: rows 16R + 4jg + i, column 16I + mr
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * R + 4 * jg + i, col = 16 * I + mr;
                    float a = accA[i] * sBeta[row];
                    float pv = accP[i];
                    if (I == R) {
                        if (col >= row) a = 0.0f;
                        if (col > row) pv = 0.0f;
                    }
                    sA[row * L::LF + col] = a;
                    store_elem(&sP[row * L::LCH + col], pv);
                }
            }
            if (DK > 64 && has_next) load_prep(c0 + CH, clen_next);
        } else {
            // ---- exact path: A and P entry by entry -----------------------------
            float Gabs[NCH];
#pragma unroll
            for (int rr = 0; rr < NRUN; ++rr) {
                const int cbase = 4 * RUN * rr + RUN * jg;
                float kk[RUN], qq[RUN];
                load_kq(rr, kk, qq);
#pragma unroll
                for (int e = 0; e < RUN; ++e) {
                    const int c = cbase + e;
                    // absolute log2 decay: block prefix + (lambda + value at the block middle)
                    Gabs[rr * RUN + e] = sFac[(F_P + R) * DK + c] + lam[rr * RUN + e] + sTot[(2 * R) * DK + c];
                    sGam[rloc * DK + c] = Gabs[rr * RUN + e];
                    if (!rvalid) { kk[e] = 0.0f; qq[e] = 0.0f; }
                }
                store_run<F32>(&sKU[rloc * L::LDK + cbase], kk);
                store_run<F32>(&sQU[rloc * L::LDK + cbase], qq);
            }
            __syncthreads();
            constexpr int NPAIR = CH * (CH + 1) / 2;
            constexpr int PPT = (NPAIR + 255) / 256;
            float resA[PPT], resP[PPT];
#pragma unroll
            for (int n = 0; n < PPT; ++n) {
                const int pidx = tid + 256 * n;
                resA[n] = 0.0f;
                resP[n] = 0.0f;
                if (pidx < NPAIR) {
                    int r = (int)((sqrtf(8.0f * pidx + 1.0f) - 1.0f) * 0.5f);
                    while ((r + 1) * (r + 2) / 2 <= pidx) ++r;
                    while (r * (r + 1) / 2 > pidx) --r;
                    const int i = pidx - r * (r + 1) / 2;
                    float sa = 0.0f, sp = 0.0f;
                    for (int c = 0; c < DK; ++c) {
                        const float f = __builtin_amdgcn_exp2f(sGam[r * DK + c] - sGam[i * DK + c]);
                        const float kic = load_elem(&sKU[i * L::LDK + c]) * f;
                        sa += load_elem(&sKU[r * L::LDK + c]) * kic;
                        sp += load_elem(&sQU[r * L::LDK + c]) * kic;
                    }
                    resA[n] = (i < r) ? sa * sBeta[r] : 0.0f;
                    resP[n] = sp;
                }
            }
            __syncthreads();
#pragma unroll
            for (int n = 0; n < PPT; ++n) {
                const int pidx = tid + 256 * n;
                if (pidx < NPAIR) {
                    int r = (int)((sqrtf(8.0f * pidx + 1.0f) - 1.0f) * 0.5f);
                    while ((r + 1) * (r + 2) / 2 <= pidx) ++r;
                    while (r * (r + 1) / 2 > pidx) --r;
                    const int i = pidx - r * (r + 1) / 2;
                    sA[r * L::LF + i] = resA[n];
                    store_elem(&sP[r * L::LCH + i], resP[n]);
                }
            }
            // zero the strict upper part of the diagonal 16x16 blocks of P
            for (int idx = tid; idx < CH * 16; idx += 256) {
                const int r = idx / 16, c = 16 * (r / 16) + (idx % 16);
                if (c > r) store_elem(&sP[r * L::LCH + c], 0.0f);
            }
#pragma unroll
            for (int rr = 0; rr < NRUN; ++rr) {
                const int cbase = 4 * RUN * rr + RUN * jg;
                float kk[RUN], qq[RUN], ku[RUN], qu[RUN], kr[RUN];
                load_kq(rr, kk, qq);
#pragma unroll
                for (int e = 0; e < RUN; ++e) {
                    const int c = cbase + e;
                    const float kv = rvalid ? kk[e] : 0.0f, qv = rvalid ? qq[e] : 0.0f;
                    const float Ga = Gabs[rr * RUN + e];
                    const float up = __builtin_amdgcn_exp2f(Ga);
                    ku[e] = -kv * up;
                    qu[e] = qv * up;
                    kr[e] = kv * __builtin_amdgcn_exp2f(sFac[(F_P + 4) * DK + c] - Ga);
                }
                store_run<F32>(&sKU[rloc * L::LDK + cbase], ku);
                store_run<F32>(&sQU[rloc * L::LDK + cbase], qu);
                if constexpr (F32) {
                    // K_right itself, row-major (read with factor 1)
                    store_run<F32>(&sKB[rloc * L::LDK + cbase], kr);
                } else {
#pragma unroll
                    for (int e = 0; e < RUN; ++e) store_elem(&sKRt[(cbase + e) * L::LCH + rloc], kr[e]);
                }
            }
            if (has_next) load_prep(c0 + CH, clen_next);
        }
        __syncthreads();

        // ================= A5: T = (I + A)^{-1}, T' = T Diag(beta) ===========
        {
            // diagonal block R by forward substitution; lane column mr
            float tcol[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == mr) ? 1.0f : 0.0f;
                const float *arow = &sA[(16 * R + r) * L::LF + 16 * R];
#pragma unroll
                for (int i = 0; i < r; ++i) acc -= arow[i] * tcol[i];
                tcol[r] = acc;
            }
            if (jg == 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sTf[(16 * R + r) * L::LF + 16 * R + mr] = tcol[r];
            }
        }
        __syncthreads();
        // off-diagonal blocks by distance d = R - I; wave R computes (R, R - d)
        for (int d = 1; d < 4; ++d) {
            if (R >= d) {
                const int I = R - d;
                f32x4 Mx = {0.f, 0.f, 0.f, 0.f};
                for (int J = I; J < R; ++J) {
                    // Mx += A[R,J] T[J,I]
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const float av = sA[(16 * R + mr) * L::LF + 16 * J + 4 * jg + s];
                        const float bv = F32 ? sTf[t_at<L::LF>(J, I, 4 * jg + s, mr)]
                                             : sTf[(16 * J + 4 * jg + s) * L::LF + 16 * I + mr];
                        Mx = mfma_f32(av, bv, Mx);
                    }
                }
                // T[R,I] = -T[R,R] Mx  (Mx accumulator is the B operand: k = 4jg + s)
                f32x4 Tx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const float av = sTf[(16 * R + mr) * L::LF + 16 * R + 4 * jg + s];
                    Tx = mfma_f32(av, Mx[s], Tx);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (F32) sTf[t_at<L::LF>(R, I, 4 * jg + i, mr)] = -Tx[i];
                    else sTf[(16 * R + 4 * jg + i) * L::LF + 16 * I + mr] = -Tx[i];
                }
            }
            __syncthreads();
        }
        // (fp32: each thread reads a diagonal or upper position and writes the
        // same diagonal position or a lower one, so no element is read by one
        // thread after another has overwritten it)
        for (int idx = tid; idx < CH * CH; idx += 256) {
            const int r = idx / CH, c = idx % CH;
            if ((c >> 4) <= (r >> 4)) {
                const float t = F32 ? sTf[t_at<L::LF>(r >> 4, c >> 4, r & 15, c & 15)] : sTf[r * L::LF + c];
                store_elem(&sTp[r * L::LCH + c], t * sBeta[c]);
            }
        }
        __syncthreads();

        // ================= B: state strips ===================================
        in_t *obase = go + ((size_t)(t0 + c0) * H + head) * DV + col0;
#pragma unroll
        for (int s = 0; s < NSTRIP; ++s) {
            const uint32_t co = 16 * (w + 4 * s) + mr;
            frag_t sf[NRUN];
#pragma unroll
            for (int rr = 0; rr < NRUN; ++rr) sf[rr] = acc_frag<F32>(S[s], rr);

            // X = V - K_up S (sKU holds -K_up), O1 = Q_up S: 4 tiles in rowmap order
            f32x4 X[4], O[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = rowmap<RUN>(tt / TPR, tt % TPR, 4 * jg + i);
                    const float vv = F32 ? __uint_as_float(rawv[s][4 * tt + i])
                                         : __uint_as_float(rawv[s][4 * tt + i] << 16);
                    X[tt][i] = row < clen ? vv : 0.0f;
                    O[tt][i] = 0.0f;
                }
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const int row = rowmap<RUN>(tt / TPR, tt % TPR, mr);
#pragma unroll
                for (int rr = 0; rr < NRUN; ++rr) {
                    const int kc = 4 * RUN * rr + RUN * jg;
                    const frag_t fa = *reinterpret_cast<const frag_t *>(&sKU[row * L::LDK + kc]);
                    const frag_t fq = *reinterpret_cast<const frag_t *>(&sQU[row * L::LDK + kc]);
                    X[tt] = mma_run<F32>(X[tt], fa, sf[rr]);
                    O[tt] = mma_run<F32>(O[tt], fq, sf[rr]);
                }
            }
            // U = T' X  (T' lower triangular: run rr needed only for rr <= run of the tile)
            constexpr int CRUN = CH / (4 * RUN);   // runs over the chunk dimension
            frag_t xf[CRUN];
#pragma unroll
            for (int rr = 0; rr < CRUN; ++rr) xf[rr] = acc_frag<F32>(X, rr);
            f32x4 U[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const int trun = tt / TPR;
                const int row = rowmap<RUN>(trun, tt % TPR, mr);
                f32x4 au = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int rr = 0; rr < CRUN; ++rr) {
                    if (rr <= trun) {
                        const frag_t fa = *reinterpret_cast<const frag_t *>(&sTp[row * L::LCH + 4 * RUN * rr + RUN * jg]);
                        au = mma_run<F32>(au, fa, xf[rr]);
                    }
                }
                U[tt] = au;
            }
            frag_t uf[CRUN];
#pragma unroll
            for (int rr = 0; rr < CRUN; ++rr) uf[rr] = acc_frag<F32>(U, rr);
            // O = O1 + P U
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const int trun = tt / TPR;
                const int row = rowmap<RUN>(trun, tt % TPR, mr);
#pragma unroll
                for (int rr = 0; rr < CRUN; ++rr) {
                    if (rr <= trun) {
                        const frag_t fa = *reinterpret_cast<const frag_t *>(&sP[row * L::LCH + 4 * RUN * rr + RUN * jg]);
                        O[tt] = mma_run<F32>(O[tt], fa, uf[rr]);
                    }
                }
            }
            // S = Diag(gamma) S + K_right^T U
#pragma unroll
            for (int tt = 0; tt < NKT; ++tt) {
                const int rho = tt / TPR, h = tt % TPR;
                const float4 gm = *reinterpret_cast<const float4 *>(&sFac[F_GAM * DK + rowmap<RUN>(rho, h, 4 * jg)]);
                S[s][tt][0] *= gm.x;
                S[s][tt][1] *= gm.y;
                S[s][tt][2] *= gm.z;
                S[s][tt][3] *= gm.w;
                const int chrow = rowmap<RUN>(rho, h, mr);
#pragma unroll
                for (int rr = 0; rr < CRUN; ++rr) {
                    frag_t fa;
                    if constexpr (F32) {
                        // K_right = k b e^{Gamma_last - Gamma_mid(rr)} on run rr's rows
                        // (K_right itself on the exact path)
                        const float fz = slow ? 1.0f : sFac[(F_Z + rr) * DK + chrow];
#pragma unroll
                        for (int e = 0; e < 4; ++e) fa[e] = sKB[(16 * rr + 4 * jg + e) * L::LDK + chrow] * fz;
                    } else {
                        fa = *reinterpret_cast<const frag_t *>(&sKRt[chrow * L::LCH + 4 * RUN * rr + RUN * jg]);
                    }
                    S[s][tt] = mma_run<F32>(S[s][tt], fa, uf[rr]);
                }
            }
            // store O (rows past the chunk end are not written)
            if (clen == CH) {
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t row = rowmap<RUN>(tt / TPR, tt % TPR, 4 * jg + i);
                        store_elem(obase + row * tokstride_v + co, O[tt][i]);
                    }
            } else {
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t row = rowmap<RUN>(tt / TPR, tt % TPR, 4 * jg + i);
                        if ((int)row < clen) store_elem(obase + row * tokstride_v + co, O[tt][i]);
                    }
            }
        }
        if (has_next) load_v(c0 + CH, clen_next);
        __syncthreads();
    }

    if (p.S_T && strow >= 0) {
        float *st = p.S_T + ((size_t)strow * H + head) * DK * DV + col0;
#pragma unroll
        for (int s = 0; s < NSTRIP; ++s) {
            const uint32_t co = 16 * (w + 4 * s) + mr;
#pragma unroll
            for (int tt = 0; tt < NKT; ++tt) {
                const int rho = tt / TPR, h = tt % TPR;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t row = rowmap<RUN>(rho, h, 4 * jg + i);
                    st[row * DV + co] = S[s][tt][i];
                }
            }
        }
    }
}

// Longest-first processing order of packed sequences: order[rank] = seq
// (a permutation of 0..n-1; the results do not depend on it, only the load
// balance does).  One workgroup of ORDER_THREADS threads.
//   n <= ORDER_SORT_MAX: exact order (longer first, equal lengths by index),
//     a bitonic sort of (length, index) keys in LDS: O(n log^2 n) work over
//     the threads, no global scratch.
//   larger n: a counting sort by length class (octave of the length and its
//     next three bits, 8 classes per octave, longest class first); inside a
//     class the order is whatever the atomics give.  O(n) work.
constexpr int ORDER_THREADS = 1024;
constexpr int ORDER_SORT_MAX = 8192;
constexpr int ORDER_CLASSES = 33 * 8;

__device__ __forceinline__ int length_class(int len) {
    // 0 for len <= 0; else 8 * (octave + 1) + next three bits, increasing with len
    if (len <= 0) return 0;
    const int oct = 31 - __builtin_clz((unsigned)len);
    const int frac = oct >= 3 ? (len >> (oct - 3)) & 7 : (len << (3 - oct)) & 7;
    return 8 * (oct + 1) + frac;
}

__global__ __launch_bounds__(ORDER_THREADS) void varlen_order_kernel(const int32_t *__restrict__ cu, int n,
                                                                     int32_t *__restrict__ order)
{
    __shared__ unsigned long long keys[ORDER_SORT_MAX];
    __shared__ int cls_count[ORDER_CLASSES];
    const int tid = threadIdx.x;
    if (n <= ORDER_SORT_MAX) {
        int m = 1;
        while (m < n) m <<= 1;
        // ascending order of (~length, index): longest first, ties by index;
        // padding keys sort last
        for (int i = tid; i < m; i += ORDER_THREADS) {
            if (i < n) {
                const unsigned len = (unsigned)(cu[i + 1] - cu[i]);
                keys[i] = ((unsigned long long)(~len) << 32) | (unsigned)i;
            } else {
                keys[i] = ~0ull;
            }
        }
        __syncthreads();
        for (int k = 2; k <= m; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                for (int i = tid; i < m; i += ORDER_THREADS) {
                    const int l = i ^ j;
                    if (l > i) {
                        const unsigned long long a = keys[i], b = keys[l];
                        const bool up = (i & k) == 0;
                        if ((a > b) == up) {
                            keys[i] = b;
                            keys[l] = a;
                        }
                    }
                }
                __syncthreads();
            }
        }
        for (int i = tid; i < n; i += ORDER_THREADS) order[i] = (int32_t)(keys[i] & 0xffffffffu);
        return;
    }
    for (int c = tid; c < ORDER_CLASSES; c += ORDER_THREADS) cls_count[c] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += ORDER_THREADS) atomicAdd(&cls_count[length_class(cu[i + 1] - cu[i])], 1);
    __syncthreads();
    if (tid == 0) {
        // exclusive prefix over classes, longest class first
        int run = 0;
        for (int c = ORDER_CLASSES - 1; c >= 0; --c) {
            const int cnt = cls_count[c];
            cls_count[c] = run;
            run += cnt;
        }
    }
    __syncthreads();
    for (int i = tid; i < n; i += ORDER_THREADS) {
        const int pos = atomicAdd(&cls_count[length_class(cu[i + 1] - cu[i])], 1);
        order[pos] = i;
    }
}

template <int DK, int NSTRIP, bool F32>
static hipError_t launch_chunked(const ChunkParams &p, hipStream_t stream)
{
    const int groups = (p.units + 7) / 8;
    const dim3 grid(groups * 8 * p.nslices);
    hipLaunchKernelGGL((chunked_fwd_kernel<DK, NSTRIP, F32>), grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

int cu_count()
{
    static int cached = 0;
    if (cached > 0) return cached;
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached = n;
    return n;
}

// Choose the value-slice width: whole d_v per workgroup when there are
// enough (sequence, head) units to fill the chip twice, else 64 columns.
int chunked_slice_width(int units, int dv)
{
    if (dv == 64) return 64;
    return (units >= 2 * cu_count()) ? 128 : 64;
}

hipError_t chunked_ws_launch(const void *q, const void *k, const void *v, const void *g,
                             const void *beta, int gate, int prep, const float *S0, float *S_T,
                             const int32_t *state_idx, int pool, void *o,
                             const int32_t *cu_seqlens, const int32_t *order, int nseq, int T,
                             int H, int dk, int dv, int slice_width, hipStream_t stream);

// ---- allocation-free forward ------------------------------------------------
// The forward's only scratch is the processing order of packed sequences.
// kda_fwd_chunked_noalloc keeps it in this file-scope device array instead of
// a caller's workspace: one copy per GPU, shared by every call on that GPU
// (overlapping calls on one GPU race), holding up to NOALLOC_MAX_SEQS
// entries.  Host code never passes the array's name to a kernel (in host
// code it is only a stand-in for the symbol): the device address is looked
// up once per device with hipGetSymbolAddress and kept.
constexpr int NOALLOC_MAX_SEQS = 65536;
static __device__ __align__(256) int32_t scratch[NOALLOC_MAX_SEQS];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
int32_t *g_scratch_ptr[MAX_DEVICES] = {};
}  // namespace

int noalloc_max_seqs() { return NOALLOC_MAX_SEQS; }

// Device address of this GPU's scratch array (current device), looked up on
// the first call on each device.
hipError_t noalloc_scratch(int32_t **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = static_cast<int32_t *>(ptr);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t chunked_fwd_launch(const void *q, const void *k, const void *v, const void *g,
                              const void *beta, int gate, int prep, const float *S0, float *S_T,
                              const int32_t *state_idx, int pool, void *o,
                              const int32_t *cu_seqlens, int num_seqs, int B, int T, int H,
                              int dk, int dv, bool bf16, void *workspace, hipStream_t stream)
{
    ChunkParams p;
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
    p.S0 = S0; p.S_T = S_T; p.o = o;
    p.cu_seqlens = cu_seqlens;
    p.order = nullptr;
    p.state_idx = state_idx;
    p.pool = pool;
    p.gate = gate;
    p.prep = prep;
    p.T = T; p.H = H; p.DV = dv;
    const int nseq = cu_seqlens ? num_seqs : B;
    p.units = nseq * H;
    if (p.units == 0) return hipSuccess;
    if (cu_seqlens && nseq > 1 && workspace) {
        int32_t *order = static_cast<int32_t *>(workspace);
        hipLaunchKernelGGL(varlen_order_kernel, dim3(1), dim3(ORDER_THREADS), 0, stream,
                           cu_seqlens, nseq, order);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        p.order = order;
    }
    const int dvs = chunked_slice_width(p.units, dv);
    if (bf16)   // producer / consumer kernel with 32-token chunks
        return chunked_ws_launch(q, k, v, g, beta, gate, prep, S0, S_T, state_idx, pool, o, cu_seqlens,
                                 p.order, nseq, T, H, dk, dv, dvs, stream);
    p.nslices = dv / dvs;
    const int nstrip = dvs / 64;
    // fp32 inputs: fp32 MFMA, 64-token chunks
    if (dk == 128)
        return nstrip == 2 ? launch_chunked<128, 2, true>(p, stream) : launch_chunked<128, 1, true>(p, stream);
    return nstrip == 2 ? launch_chunked<64, 2, true>(p, stream) : launch_chunked<64, 1, true>(p, stream);
}

}  // namespace kda
