// hh_distill.hip -- fused attention-weight distillation loss on the CDNA4 matrix cores.
//
// The loss of Eq. 4 (paper-graph-ui walkthrough of "The Hedgehog & the Porcupine", section 3.4,
// "The Attention Weight Distillation Loss"): for query i of one (batch, head),
//     p_ij = softmax over j <= i of q_i.k_j / sqrt(d)          (the raw q and k)
//     a_ij = phi(q_i).phi(k_j)                                  (the feature map's kernel)
//     L_i  = -sum_{j<=i} p_ij log(a_ij / sum_{m<=i} a_im)
// Since the p_ij sum to 1, L_i = -(sum_j e_ij log a_ij) / (sum_j e_ij) + log(sum_j a_ij) with
// e_ij = exp(q_i.k_j / sqrt(d) - m_i) for any m_i; the kernel keeps, per query, a running maximum
// m_i of the logits and the three sums, rescaling two of them when m_i grows (the usual one-pass
// softmax), so the n^2 weights are never stored.
//
// One workgroup of eight waves owns 128 queries of one (b,h) (16 per wave) and walks the key
// tiles of 64 up to its diagonal; each staged tile serves all eight waves.  Per 16-key block, the scores come from the matrix cores with the keys as rows
// and the queries as columns, so a lane holds one query and four keys: the per-query reductions
// run inside the lane and across the four lane groups (two shuffles).
//   Hedgehog: a = phi(q).phi(k).  The key features (2d per key, bf16 as the forward pass uses
//             them) are precomputed by the feature-map kernel, since every query tile reads them;
//             each wave maps its own 16 queries in its prologue (u = W q + b on the matrix cores,
//             W staged once per workgroup in the key-feature tile's space, then the exponentials),
//             straight into the operand registers of the weight products:
//             two 16-direction accumulator blocks give lane group g the features 4g..4g+3 and
//             16+4g..16+4g+3 of a 32-feature step, and the key features are read in that order.
//   Taylor:   a = 1 + s + s^2/2 with s = q.k, the map's closed form (section 3.4, "The Taylor
//             Exponential as a Bridge Result"), from the same product as the logits.
// The next key tile is fetched into registers while the current one is in use.
#include "hh_common.h"
#include "hh_kernels.h"

namespace hh {

namespace {
constexpr int QT = 128;  // queries per workgroup
constexpr int NT = 512;  // threads per workgroup (eight waves of 16 queries)
constexpr int KT = 64;  // keys per tile
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kSchedValu = 0x2, kSchedMfma = 0x8, kSchedDsRead = 0x100;  // scheduling-group masks
}  // namespace

template <int D, bool TAY>
struct DistillCfg {
    static constexpr int DF = TAY ? 0 : 2 * D;         // feature columns staged per key
    static constexpr int KP = D + 16;                   // row pitch of the key tile (bf16)
    static constexpr int FP = DF + 16;                  // row pitch of the key-feature tile
    static constexpr int KSD = (D + 31) / 32;           // K steps over the head dim (d = 16: half)
    static constexpr int KSF = DF / 32;                 // K steps over the features
    static constexpr int GK = KT * D / 8;               // 16-byte pieces of a key tile
    static constexpr int GF = KT * DF / 8;              // 16-byte pieces of a key-feature tile
    static constexpr int PK = (GK + NT - 1) / NT;       // pieces per thread
    static constexpr int PF = (GF + NT - 1) / NT;
};

template <int D, bool TAY>
__global__ __launch_bounds__(NT) void distill_kernel(DistillParams p) {
    using C = DistillCfg<D, TAY>;
    __shared__ __attribute__((aligned(16))) bf16_t sK[KT * C::KP];
    __shared__ __attribute__((aligned(16))) bf16_t sF[TAY ? 8 : KT * C::FP];
    const int nqt = (p.N + QT - 1) / QT;
    // The longest rows of queries (most key tiles) are dispatched first.  Workgroups go to the
    // eight XCDs round-robin (blockIdx mod 8): when the (b,h) count allows, all query tiles of one
    // (b,h) land on one XCD, so its keys and key features are fetched into that XCD's L2 once.
    int bh, qt;
    if (p.BH % 8 == 0) {
        const int nhx = p.BH / 8, k = blockIdx.x / 8;
        bh = blockIdx.x % 8 + 8 * (k % nhx);
        qt = nqt - 1 - k / nhx;
    } else {
        bh = blockIdx.x / nqt;
        qt = nqt - 1 - blockIdx.x % nqt;
    }
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 4, r16 = lane & 15;
    const size_t base = (size_t)bh * p.N;
    const int qi = QT * qt + 16 * w + r16;  // this lane's query
    const bool qok = qi < p.N;

    // Query operands (B operands: column = query, K = head dims / features), kept in registers.
    bf16x8 qop[C::KSD], fop[TAY ? 1 : C::KSF];
#pragma unroll
    for (int ks = 0; ks < C::KSD; ks++) {
        const int c0 = 32 * ks + 8 * g;
        qop[ks] = (qok && c0 < D) ? load8(p.q + (base + qi) * D + c0) : zero_bf16x8();
    }
    if (!TAY) {
        // u[l][query] for directions l = 16 mb + 4 g + rr (A: W rows, B: the query operands), then
        // feature step ks (ks < d / 32: exp(u), else exp(-u)) from direction blocks 2 (ks mod d/32)
        // and 2 (ks mod d/32) + 1
        const int h = bh % p.H;
        const bf16_t *Wh = p.W + (size_t)h * D * D;
        constexpr int WP = D + 8;  // row pitch of W in LDS (the key-feature tile is free until the first tile)
        static_assert(D * WP <= KT * C::FP, "W fits in the key-feature tile");
        stage_pieces<NT, D * D / 8>(
            tid, [&](int e) { return Wh + 8 * e; }, [&](int e) { return sF + (e / (D / 8)) * WP + 8 * (e % (D / 8)); },
            [](int) { return true; });
        __syncthreads();
        constexpr int NMB = D / 16;
        // the bias of directions 16 mb + 4 g + rr, all loads issued behind one test of the pointer
        float bq[NMB][4];
#pragma unroll
        for (int mb = 0; mb < NMB; mb++)
#pragma unroll
            for (int rr = 0; rr < 4; rr++) bq[mb][rr] = 0.0f;
        if (p.b) {
#pragma unroll
            for (int mb = 0; mb < NMB; mb++)
#pragma unroll
                for (int rr = 0; rr < 4; rr++) bq[mb][rr] = bf16_bits_to_float(p.b[(size_t)h * D + 16 * mb + 4 * g + rr]);
        }
        f32x4 u[NMB];
#pragma unroll
        for (int mb = 0; mb < NMB; mb++) {
            bf16x8 wa[C::KSD];
#pragma unroll
            for (int ks = 0; ks < C::KSD; ks++) {
                const int m0 = 32 * ks + 8 * g;
                wa[ks] = m0 < D ? load8(sF + (16 * mb + r16) * WP + m0) : zero_bf16x8();
            }
            u[mb] = zero4();
#pragma unroll
            for (int ks = 0; ks < C::KSD; ks++) u[mb] = mfma_bf16(wa[ks], qop[ks], u[mb]);
#pragma unroll
            for (int rr = 0; rr < 4; rr++) u[mb][rr] = (u[mb][rr] + bq[mb][rr]) * kLog2e;
        }
        // (d = 16: one step, exp(u) of the 16 directions then exp(-u) of the same)
        constexpr int HALF = C::KSF / 2 > 0 ? C::KSF / 2 : 1;
#pragma unroll
        for (int ks = 0; ks < C::KSF; ks++) {
            const int mb0 = D == 16 ? 0 : 2 * (ks % HALF);
            const int mb1 = D == 16 ? 0 : mb0 + 1;
            const float sg0 = D == 16 ? 1.0f : (ks < HALF ? 1.0f : -1.0f);
            const float sg1 = D == 16 ? -1.0f : sg0;
            f32x4 lo, hi;
#pragma unroll
            for (int rr = 0; rr < 4; rr++) {
                lo[rr] = exp2_fast(sg0 * u[mb0][rr]);
                hi[rr] = exp2_fast(sg1 * u[mb1][rr]);
            }
            fop[ks] = qok ? acc_pair_to_operand(lo, hi) : zero_bf16x8();
        }
    }

    // Key tiles through registers: piece e of a tile is row e / (D / 8), 16-byte column e % (D / 8).
    bf16x8 rk[C::PK], rf[TAY ? 1 : C::PF];
    auto fetch = [&](int kt) {
#pragma unroll
        for (int u = 0; u < C::PK; u++) {
            const int e = tid + NT * u;
            const int row = e / (D / 8), c8 = e % (D / 8), j = KT * kt + row;
            rk[u] = (e < C::GK && j < p.N) ? load8(p.k + (base + j) * D + 8 * c8) : zero_bf16x8();
        }
        if (!TAY) {
#pragma unroll
            for (int u = 0; u < C::PF; u++) {
                const int e = tid + NT * u;
                const int row = e / (C::DF / 8), c8 = e % (C::DF / 8), j = KT * kt + row;
                rf[u] = (e < C::GF && j < p.N) ? load8(p.phi_k + (base + j) * C::DF + 8 * c8) : zero_bf16x8();
            }
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int u = 0; u < C::PK; u++) {
            const int e = tid + NT * u;
            if (e < C::GK) store8(sK + (e / (D / 8)) * C::KP + 8 * (e % (D / 8)), rk[u]);
        }
        if (!TAY) {
            // key features stored in the K order of the query operands: within each 32-feature
            // group, the 4-feature units 0..3 go to slots 0, 2, 4, 6 and units 4..7 to slots 1, 3,
            // 5, 7, so that the 16-byte read of lane group g holds features 4g.. and 16+4g..
#pragma unroll
            for (int u = 0; u < C::PF; u++) {
                const int e = tid + NT * u;
                if (e < C::GF) {
                    const int row = e / (C::DF / 8), c8 = e % (C::DF / 8);
                    const int grp = c8 >> 2, lu = 2 * (c8 & 3);                 // local units lu, lu + 1
                    const int s0 = lu < 4 ? 2 * lu : 2 * (lu - 4) + 1, s1 = lu + 1 < 4 ? 2 * (lu + 1) : 2 * (lu - 3) + 1;
                    bf16_t *dst = sF + row * C::FP + 32 * grp;
                    store4(dst + 4 * s0, __builtin_shufflevector(rf[u], rf[u], 0, 1, 2, 3));
                    store4(dst + 4 * s1, __builtin_shufflevector(rf[u], rf[u], 4, 5, 6, 7));
                }
            }
        }
    };

    // Per query (this lane's share of the keys): running maximum of the logits in log2 units, and
    // the sums of e = 2^(logit - m), of e log2(a), and of a.
    const float lscale = kLog2e * rsqrtf((float)D);
    float m = -1.0e30f, l = 0.0f, t = 0.0f, r = 0.0f;

    // The products of the staged tile: raw scores s (A operands: key rows 16 nb + r16 of the tile;
    // lane holds query r16, keys 4 g + rr of block nb) and the weights a.  Each group of operand
    // reads is issued before its products, so the reads overlap one another; vector work (the
    // update of the previous tile) may be scheduled between them.
    auto products = [&](float (&x)[4][4], float (&av)[4][4], bool fenced) {
#pragma unroll
        for (int n2 = 0; n2 < 2; n2++) {  // two key blocks per group of reads
            bf16x8 ko[2][C::KSD];
#pragma unroll
            for (int h = 0; h < 2; h++)
#pragma unroll
                for (int ks = 0; ks < C::KSD; ks++) {
                    const int c0 = 32 * ks + 8 * g;
                    ko[h][ks] = c0 < D ? load8(sK + (16 * (2 * n2 + h) + r16) * C::KP + c0) : zero_bf16x8();
                }
            if (fenced) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const int nb = 2 * n2 + h;
                f32x4 sv = zero4();
#pragma unroll
                for (int ks = 0; ks < C::KSD; ks++) sv = mfma_bf16(ko[h][ks], qop[ks], sv);
#pragma unroll
                for (int rr = 0; rr < 4; rr++) {
                    x[nb][rr] = sv[rr];
                    if (TAY) av[nb][rr] = fmaf(sv[rr], fmaf(0.5f, sv[rr], 1.0f), 1.0f);
                }
            }
        }
        if (!TAY) {
#pragma unroll
            for (int nb = 0; nb < 4; nb++) {  // one key block per group of reads
                bf16x8 fo[TAY ? 1 : C::KSF];
#pragma unroll
                for (int ks = 0; ks < C::KSF; ks++) fo[ks] = load8(sF + (16 * nb + r16) * C::FP + 32 * ks + 8 * g);
                if (fenced) __builtin_amdgcn_sched_barrier(0);
                f32x4 aa = zero4();
#pragma unroll
                for (int ks = 0; ks < C::KSF; ks++) aa = mfma_bf16(fo[ks], fop[ks], aa);
#pragma unroll
                for (int rr = 0; rr < 4; rr++) av[nb][rr] = aa[rr];
            }
        }
    };
    // The one-pass softmax update with one tile's scores: new maximum (across the four lane groups
    // of a query), rescaled sums, then the tile's terms.  Keys of a masked tile past the query or
    // past the end get s = -inf (e = 0) and a = 0; the log of the stand-in 1 keeps 0 log 0 from a
    // NaN.  A tile with no masked key takes the branch-free form.
    auto update = [&](float (&x)[4][4], float (&av)[4][4], bool masked, int kt) {
        float mb = -1.0e30f;
        if (masked) {
            const int kbase = KT * kt + 4 * g;
#pragma unroll
            for (int nb = 0; nb < 4; nb++)
#pragma unroll
                for (int rr = 0; rr < 4; rr++) {
                    const int j = kbase + 16 * nb + rr;
                    if (!(j <= qi && j < p.N)) {
                        x[nb][rr] = -1.0e30f;
                        av[nb][rr] = 0.0f;
                    }
                }
        }
#pragma unroll
        for (int nb = 0; nb < 4; nb++)
#pragma unroll
            for (int rr = 0; rr < 4; rr++) mb = fmaxf(mb, x[nb][rr]);
        mb = fmaxf(mb, __shfl_xor(mb, 16));
        mb = fmaxf(mb, __shfl_xor(mb, 32));
        const float mn = fmaxf(m, mb * lscale);  // lscale > 0: the maximum of the scaled logits
        const float sc = exp2_fast(m - mn);
        l *= sc;
        t *= sc;
        m = mn;
#pragma unroll
        for (int nb = 0; nb < 4; nb++)
#pragma unroll
            for (int rr = 0; rr < 4; rr++) {
                const float e = exp2_fast(fmaf(x[nb][rr], lscale, -m));
                l += e;
                r += av[nb][rr];
                t = fmaf(e, __builtin_amdgcn_logf(masked ? (av[nb][rr] > 0.0f ? av[nb][rr] : 1.0f) : av[nb][rr]), t);
            }
    };
    const int nkt = min(QT * qt + QT - 1, p.N - 1) / KT + 1;
    const int nfull = min(min((QT * qt + 1) / KT, p.N / KT), nkt);
    auto next_tile = [&](int kt) {
        __syncthreads();  // the previous tile is no longer read
        stage();
        __syncthreads();
        if (kt + 1 < nkt) fetch(kt + 1);
    };

    // Key tiles up to the one holding the workgroup's last query (or the sequence's last key).
    // The leading tiles with no masked key (below the diagonal and inside the sequence) run as a
    // software pipeline: the products of tile kt are issued alongside the update with tile kt - 1,
    // so each wave keeps the matrix and vector pipes busy at once; the masked tiles follow.
    fetch(0);
    int kt = 0;
    if (nfull > 0) {
        float xp[4][4], ap[4][4];
        next_tile(0);
        products(xp, ap, true);
        for (kt = 1; kt < nfull; kt++) {
            next_tile(kt);
            float x[4][4], av[4][4];
            products(x, av, false);
            update(xp, ap, false, kt - 1);
#pragma unroll
            for (int nb = 0; nb < 4; nb++)
#pragma unroll
                for (int rr = 0; rr < 4; rr++) {
                    xp[nb][rr] = x[nb][rr];
                    ap[nb][rr] = av[nb][rr];
                }
            // Issue order: four operand reads, then each product with two vector instructions of
            // the update beside it and the next operand read (measured against three and four
            // vector instructions and two, eight and sixteen reads ahead).
            if (D == 128) {
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
                for (int i = 0; i < 48; i++) {
                    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(kSchedValu, 2, 0);
                    if (i < 44) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
                }
            }
        }
        update(xp, ap, false, nfull - 1);
    }
    for (; kt < nkt; kt++) {
        next_tile(kt);
        float x[4][4], av[4][4];
        products(x, av, true);
        update(x, av, true, kt);
    }
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    t += __shfl_xor(t, 16);
    t += __shfl_xor(t, 32);
    r += __shfl_xor(r, 16);
    r += __shfl_xor(r, 32);
    if (g == 0 && qok) p.loss[base + qi] = (__builtin_amdgcn_logf(r) - t / l) * kLn2;
}

hipError_t launch_distill(int map, int d, const DistillParams &p, int BH, hipStream_t st) {
    const int nqt = (p.N + QT - 1) / QT;
    const dim3 grid((unsigned)((long)BH * nqt)), block(NT);
    if (map == 1) {
        if (d != 16) return hipErrorInvalidValue;
        hipLaunchKernelGGL((distill_kernel<16, true>), grid, block, 0, st, p);
        return hipGetLastError();
    }
    switch (d) {
    case 16: hipLaunchKernelGGL((distill_kernel<16, false>), grid, block, 0, st, p); break;
    case 32: hipLaunchKernelGGL((distill_kernel<32, false>), grid, block, 0, st, p); break;
    case 64: hipLaunchKernelGGL((distill_kernel<64, false>), grid, block, 0, st, p); break;
    case 128: hipLaunchKernelGGL((distill_kernel<128, false>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace hh
