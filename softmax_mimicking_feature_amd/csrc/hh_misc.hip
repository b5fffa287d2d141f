// hh_misc.hip -- the smaller libhh kernels: Taylor segment prefix, empty-sequence state,
// the fp32 token-by-token path, the decode step and the vector-unit feature map.
//
// Feature maps (paper-graph-ui walkthrough of "The Hedgehog & the Porcupine"):
//   Hedgehog (section 3.4, "The Hedgehog MLP Feature Map", Choices 1 and 3):
//       u_l = b_l + sum_m W[l][m] x_m,   phi = [exp(u_0..u_{d-1}), exp(-u_0..-u_{d-1})]
//   Taylor (section 3.4, "The Taylor Exponential as a Bridge Result"):
//       phi = [1, x_0..x_{d-1}, x_a x_c / sqrt(2) for a, c in [d], row-major]
// Running sums and read-out: Eq. 2 with S_i, z_i (section 2; section 3.4 "Complexity Analysis").
#include "hh_common.h"
#include "hh_kernels.h"

namespace hh {

// ----------------------------------------------------------------------------------------
// Internal rows of the Taylor state in the chunked kernels: a packed symmetric basis of 160
// rows (1 + 16 + 136 features, padded).  Row p < 16: the linear feature x_p (canonical row
// 1 + p).  Row 16 (1 + o) + p, o = 0..7: the pair (p, c = p + o mod 16); o = 0 is the
// diagonal x_p^2 / sqrt(2) (canonical row 17 + 17 p), o > 0 the off-diagonal feature x_p x_c,
// which carries both canonical rows (p, c) and (c, p), each x_p x_c / sqrt(2).  Rows 144 + p:
// the pair (p, p + 8) for p < 8, the constant feature at p = 8 (canonical row 0), zero above.
// Value of internal row r of a canonical state X (element (row, col) at X[row * ld + col]):
// a pair row is (X_pc + X_cp) / sqrt(2), which keeps every query's read-out of X unchanged.
__device__ __forceinline__ float taylor_packed_value(const float *X, int r, int col, int ld) {
    constexpr float kInvSqrt2 = 0.70710678118654752f;
    if (r < 16) return X[(size_t)(1 + r) * ld + col];
    int p, c;
    if (r < 144) {
        const int o = r / 16 - 1;
        p = r % 16;
        if (o == 0) return X[(size_t)(17 + 17 * p) * ld + col];
        c = (p + o) & 15;
    } else {
        p = r - 144;
        if (p == 8) return X[col];
        if (p > 8) return 0.0f;
        c = p + 8;
    }
    return (X[(size_t)(17 + 16 * p + c) * ld + col] + X[(size_t)(17 + 16 * c + p) * ld + col]) * kInvSqrt2;
}

__global__ void prefix_kernel(PrefixParams p) {
    const long per = (long)p.dpi * p.d + p.dpi;
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)p.BH * per) return;
    const int bh = (int)(idx / per);
    const long e = idx % per;
    const bool isS = e < (long)p.dpi * p.d;
    const int row = isS ? (int)(e / p.d) : (int)(e - (long)p.dpi * p.d);
    const int col = isS ? (int)(e % p.d) : 0;
    float *base;
    long stride;
    if (isS) {
        stride = (long)p.dpi * p.d;
        base = p.S_ws + (size_t)bh * p.nseg * stride + e;
    } else {
        stride = p.dpi;
        base = p.z_ws + (size_t)bh * p.nseg * stride + row;
    }
    float run = 0.0f;
    if (p.S0) {
        if (p.map == 0) run = isS ? p.S0[((size_t)bh * p.dpc + row) * p.d + col] : p.z0[(size_t)bh * p.dpc + row];
        else run = isS ? taylor_packed_value(p.S0 + (size_t)bh * p.dpc * p.d, row, col, p.d)
                       : taylor_packed_value(p.z0 + (size_t)bh * p.dpc, row, 0, 1);
    }
    // Segments go in groups of G: all loads of a group are issued before its stores, so that a
    // thread waits for memory once per group rather than once per segment.
    constexpr int G = 16;
    if (p.mode == 0) {  // exclusive prefix; the last segment's own aggregate is never needed
        for (int s0 = 0; s0 < p.nseg; s0 += G) {
            float a[G];
#pragma unroll
            for (int j = 0; j < G; j++) a[j] = (s0 + j < p.nseg - 1) ? base[(s0 + j) * stride] : 0.0f;
#pragma unroll
            for (int j = 0; j < G; j++)
                if (s0 + j < p.nseg) {
                    base[(s0 + j) * stride] = run;
                    run += a[j];
                }
        }
    } else {  // total over all segments into slot 0
        for (int s0 = 0; s0 < p.nseg; s0 += G) {
            float a[G];
#pragma unroll
            for (int j = 0; j < G; j++) a[j] = (s0 + j < p.nseg) ? base[(s0 + j) * stride] : 0.0f;
#pragma unroll
            for (int j = 0; j < G; j++) run += a[j];
        }
        base[0] = run;
    }
}

hipError_t launch_prefix(const PrefixParams &p, hipStream_t st) {
    const long per = (long)p.dpi * p.d + p.dpi;
    const long total = (long)p.BH * per;
    const int nt = 256;
    hipLaunchKernelGGL(prefix_kernel, dim3((unsigned)((total + nt - 1) / nt)), dim3(nt), 0, st, p);
    return hipGetLastError();
}

__global__ void state_copy_kernel(const float *S0, const float *z0, float *S_out, float *z_out, long nS, long nz) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < nS) S_out[i] = S0 ? S0[i] : 0.0f;
    else if (i < nS + nz) z_out[i - nS] = z0 ? z0[i - nS] : 0.0f;
}

hipError_t launch_state_copy(const float *S0, const float *z0, float *S_out, float *z_out, long nS, long nz,
                             hipStream_t st) {
    const long total = nS + nz;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, S0, z0, S_out,
                       z_out, nS, nz);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------------------
// Feature value f of token x (fp32), x already in shared memory.  For the softmax maps this is
// the logit (+-w_l.x); softmax_halves turns a token's logits into features afterwards.
template <typename LoadW>
__device__ __forceinline__ float feature_value(int map, int d, int f, const float *x, LoadW wrow, float bias_l,
                                               const QuadCoef &qc) {
    if (map != HH_MAP_TAYLOR2_ && map != HH_MAP_QUADRATIC_) {
        const int l = f < d ? f : f - d;
        float u = bias_l;
        for (int m = 0; m < d; m++) u = fmaf(wrow(l, m), x[m], u);
        const float su = f < d ? u : -u;
        return (map == HH_MAP_HEDGEHOG_SOFTMAX_ || map == HH_MAP_SOFTMAX_) ? su : expf(su);
    }
    // quadratic kernels a + b s + c s^2: [sqrt a, sqrt b x, sqrt c x_a x_c] (Taylor: 1, 1, 1/2)
    if (f == 0) return qc.sa;
    if (f <= d) return x[f - 1] * qc.sb;
    const int q = f - 1 - d;
    return x[q / d] * x[q % d] * qc.sc;
}

__device__ __forceinline__ bool quadratic_family(int map) { return map == HH_MAP_TAYLOR2_ || map == HH_MAP_QUADRATIC_; }

// Softmax over each half (d logits) of a token's feature vector in shared memory, in place;
// executed by one wave (lane l handles entries l and l + 64 of each half, d <= 128).
__device__ __forceinline__ void softmax_halves(float *sf, int d, int halves, int lane) {
    for (int hf = 0; hf < halves; hf++) {
        float *x = sf + hf * d;
        float v0 = lane < d ? x[lane] : -INFINITY, v1 = lane + 64 < d ? x[lane + 64] : -INFINITY;
        float mx = fmaxf(v0, v1);
        for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        const float e0 = lane < d ? expf(v0 - mx) : 0.0f, e1 = lane + 64 < d ? expf(v1 - mx) : 0.0f;
        float sum = e0 + e1;
        for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
        if (lane < d) x[lane] = e0 / sum;
        if (lane + 64 < d) x[lane + 64] = e1 / sum;
    }
}

__device__ __forceinline__ bool is_softmax_map(int map) {
    return map == HH_MAP_HEDGEHOG_SOFTMAX_ || map == HH_MAP_SOFTMAX_;
}

__device__ __forceinline__ float ld(const void *p, size_t i, int dtype) {
    return dtype == 1 ? bf16_bits_to_float(reinterpret_cast<const bf16_t *>(p)[i])
                      : reinterpret_cast<const float *>(p)[i];
}
__device__ __forceinline__ void st(void *p, size_t i, float v, int dtype) {
    if (dtype == 1) reinterpret_cast<bf16_t *>(p)[i] = float_to_bf16_bits(v);
    else reinterpret_cast<float *>(p)[i] = v;
}

// fp32 path.  One workgroup per (b,h); thread t owns state elements e = t + 256 m of
// S [dp][d] (all in column t % d, since 256 is a multiple of d), kept in registers.
constexpr int kSeqThreads = 256;
constexpr int kSeqMaxE = 128;     // dp * d <= 256 * 128
constexpr int kMaxDp = 288;

__global__ __launch_bounds__(kSeqThreads) void seq_f32_kernel(SeqParams p) {
    __shared__ float sk[128], sq[128], sv[128];
    __shared__ float sfk[kMaxDp], sfq[kMaxDp], sz[kMaxDp];
    __shared__ float sred[kSeqThreads];
    const int bh = blockIdx.x, h = bh % p.H, t = threadIdx.x;
    const int d = p.d, dp = p.dp, nE = dp * d;
    const bool quad = quadratic_family(p.map);
    const float *Wh = (p.W && !quad) ? p.W + (size_t)h * d * d : nullptr;
    const QuadCoef qc = quad_coef(p.map == HH_MAP_QUADRATIC_ ? p.W : nullptr, h);
    const float *bhp = p.b ? p.b + (size_t)h * d : nullptr;
    auto wrow = [&](int l, int m) { return Wh[l * d + m]; };
    const size_t seq = (size_t)bh * p.N * d;

    float S[kSeqMaxE];
#pragma unroll
    for (int m = 0; m < kSeqMaxE; m++) {
        const int e = t + kSeqThreads * m;
        S[m] = (e < nE && p.S0) ? p.S0[(size_t)bh * nE + e] : 0.0f;
    }
    for (int f = t; f < dp; f += kSeqThreads) sz[f] = p.z0 ? p.z0[(size_t)bh * dp + f] : 0.0f;
    const int ncol = t % d;

    // pass over keys (causal: interleaved with queries; bidirectional: all keys first)
    for (int pass = 0; pass < (p.causal ? 1 : 2); pass++) {
        const bool do_update = p.causal || pass == 0;
        const bool do_read = p.causal || pass == 1;
        for (int i = 0; i < p.N; i++) {
            __syncthreads();
            if (t < d) {
                sk[t] = p.k[seq + (size_t)i * d + t];
                sq[t] = p.q[seq + (size_t)i * d + t];
                sv[t] = p.v[seq + (size_t)i * d + t];
            }
            __syncthreads();
            for (int f = t; f < dp; f += kSeqThreads) {
                const int l = f < d ? f : f - d;
                const float bl = ((p.map == HH_MAP_HEDGEHOG_ || p.map == HH_MAP_EXP_) && bhp) ? bhp[l] : 0.0f;
                if (do_update) sfk[f] = feature_value(p.map, d, f, sk, wrow, bl, qc);
                if (do_read) sfq[f] = feature_value(p.map, d, f, sq, wrow, bl, qc);
            }
            __syncthreads();
            if (is_softmax_map(p.map)) {
                const int halves = p.map == HH_MAP_HEDGEHOG_SOFTMAX_ ? 2 : 1;
                if (t < 64 && do_update) softmax_halves(sfk, d, halves, t);
                if (t >= 64 && t < 128 && do_read) softmax_halves(sfq, d, halves, t - 64);
                __syncthreads();
            }
            if (do_update) {
#pragma unroll
                for (int m = 0; m < kSeqMaxE; m++) {
                    const int e = t + kSeqThreads * m;
                    if (e < nE) S[m] = fmaf(sfk[e / d], sv[ncol], S[m]);
                }
                for (int f = t; f < dp; f += kSeqThreads) sz[f] += sfk[f];
            }
            if (do_read) {
                float part = 0.0f;
#pragma unroll
                for (int m = 0; m < kSeqMaxE; m++) {
                    const int e = t + kSeqThreads * m;
                    if (e < nE) part = fmaf(sfq[e / d], S[m], part);
                }
                sred[t] = part;
                __syncthreads();
                if (t < d) {
                    float num = 0.0f;
                    for (int u = t; u < kSeqThreads; u += d) num += sred[u];
                    float den = 0.0f;
                    for (int f = 0; f < dp; f++) den = fmaf(sfq[f], sz[f], den);
                    p.y[seq + (size_t)i * d + t] = num / den;
                }
            }
        }
    }
    __syncthreads();
    if (p.S_out) {
#pragma unroll
        for (int m = 0; m < kSeqMaxE; m++) {
            const int e = t + kSeqThreads * m;
            if (e < nE) p.S_out[(size_t)bh * nE + e] = S[m];
        }
        for (int f = t; f < dp; f += kSeqThreads) p.z_out[(size_t)bh * dp + f] = sz[f];
    }
}

hipError_t launch_seq_f32(const SeqParams &p, int BH, hipStream_t st) {
    hipLaunchKernelGGL(seq_f32_kernel, dim3(BH), dim3(kSeqThreads), 0, st, p);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------------------
// Decode step.  One workgroup per (b,h): features of the new q and k, then one streaming
// pass over S [dp][d] (read, add phi(k) v^T, write back, accumulate phi(q)^T S), float4
// per thread.  Thread t always touches column quad t % (d/4).  Loads leave in the order they
// are needed: the token's q, k, v and this thread's part of W, then the state pieces.  All
// workgroups request their state at once, so a load queued behind them would arrive only
// with the last of them, and the feature maps, and every write of S after them, would wait.
#ifndef HH_DEC_THREADS
#define HH_DEC_THREADS 256
#endif
constexpr int kDecThreads = HH_DEC_THREADS;
constexpr int kDecHeld = 32;  // state pieces per thread fetched up front (all of them for d = 128)
constexpr int kDecWPieces = 8;  // 16-byte pieces of W per thread held in registers (d = 128: 8)

__global__ __launch_bounds__(kDecThreads) void decode_kernel(DecodeParams p) {
    __shared__ float sq[128], sk[128], sv[128];
    __shared__ float sfq[kMaxDp], sfk[kMaxDp];
    __shared__ f32x4 sred[kDecThreads];
    __shared__ float sden[kDecThreads / 64];
    const int bh = blockIdx.x, h = bh % p.H, t = threadIdx.x;
    const int d = p.d, dp = p.dp, dt = p.dtype;
    // This thread's part of S (16-byte pieces e4 = t + kDecThreads i) is requested before the
    // feature maps are computed, so that the state read overlaps them; states with more pieces
    // than kDecHeld per thread take the streaming loop below for the rest.
    const int q4 = d / 4;
    const int n4 = dp * q4;
    f32x4 *S4 = reinterpret_cast<f32x4 *>(p.S + (size_t)bh * dp * d);
    float xq = 0.0f, xk = 0.0f, xv = 0.0f;
    if (t < d) {
        xq = ld(p.q, (size_t)bh * d + t, dt);
        xk = ld(p.k, (size_t)bh * d + t, dt);
        xv = ld(p.v, (size_t)bh * d + t, dt);
    }
    const void *W = p.W;
    const size_t woff = (size_t)h * d * d;
    // u = W x for q and k together: kDecThreads / d consecutive threads share a row of W and
    // read contiguous pieces of it (held in registers when they are whole 16-byte pieces of a
    // bf16 W), then combine their partial dot products
    const int tpr = kDecThreads / d < d ? kDecThreads / d : d;
    const int l = t / tpr, part = t % tpr, ept = d / tpr;
    const size_t ro = woff + (size_t)(l < d ? l : 0) * d + (size_t)part * ept;
    const bool wreg_path = !quadratic_family(p.map) && dt == 1 && ept % 8 == 0 && ept / 8 <= kDecWPieces;
    bf16x8 wreg[kDecWPieces];
    if (wreg_path && l < d) {
        const bf16x8 *wr = reinterpret_cast<const bf16x8 *>(reinterpret_cast<const bf16_t *>(W) + ro);
#pragma unroll
        for (int j = 0; j < kDecWPieces; j++)
            if (j < ept / 8) wreg[j] = wr[j];
    }
    f32x4 held[kDecHeld];
#pragma unroll
    for (int i = 0; i < kDecHeld; i++) {
        const int e4 = t + kDecThreads * i;
        if (e4 < n4) held[i] = __builtin_nontemporal_load(S4 + e4);
    }
    if (t < d) {
        sq[t] = xq;
        sk[t] = xk;
        sv[t] = xv;
    }
    __syncthreads();
    if (!quadratic_family(p.map)) {
        float uq = 0.0f, uk = 0.0f;
        if (l >= d) {
            // spare threads (more threads than d rows x d elements): nothing to add
        } else if (wreg_path) {
#pragma unroll
            for (int j = 0; j < kDecWPieces; j++) {
                if (j >= ept / 8) break;
                const bf16x8 wv = wreg[j];
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const float wf = (float)wv[e];
                    uq = fmaf(wf, sq[part * ept + 8 * j + e], uq);
                    uk = fmaf(wf, sk[part * ept + 8 * j + e], uk);
                }
            }
        } else {
            for (int m = 0; m < ept; m++) {
                const float wf = ld(W, ro + m, dt);
                uq = fmaf(wf, sq[part * ept + m], uq);
                uk = fmaf(wf, sk[part * ept + m], uk);
            }
        }
        for (int o = tpr / 2; o > 0; o >>= 1) {
            uq += __shfl_xor(uq, o);
            uk += __shfl_xor(uk, o);
        }
        if (part == 0 && l < d) {
            const float bl = p.b ? ld(p.b, (size_t)h * d + l, dt) : 0.0f;
            if (p.map == HH_MAP_HEDGEHOG_) {
                sfq[l] = expf(uq + bl);
                sfq[d + l] = expf(-(uq + bl));
                sfk[l] = expf(uk + bl);
                sfk[d + l] = expf(-(uk + bl));
            } else if (p.map == HH_MAP_EXP_) {
                sfq[l] = expf(uq + bl);
                sfk[l] = expf(uk + bl);
            } else {  // softmax maps: logits first (no bias), normalised below
                sfq[l] = uq;
                sfk[l] = uk;
                if (p.map == HH_MAP_HEDGEHOG_SOFTMAX_) {
                    sfq[d + l] = -uq;
                    sfk[d + l] = -uk;
                }
            }
        }
        if (is_softmax_map(p.map)) {
            __syncthreads();
            const int halves = p.map == HH_MAP_HEDGEHOG_SOFTMAX_ ? 2 : 1;
            if (t < 64) softmax_halves(sfq, d, halves, t);
            else if (t < 128) softmax_halves(sfk, d, halves, t - 64);
        }
    } else {
        // quadratic kernels: W holds the generalised map's fp32 coefficients (null for Taylor)
        auto wrow = [&](int, int) { return 0.0f; };
        const QuadCoef qc = quad_coef(p.map == HH_MAP_QUADRATIC_ ? reinterpret_cast<const float *>(W) : nullptr, h);
        for (int f = t; f < dp; f += kDecThreads) {
            sfk[f] = feature_value(p.map, d, f, sk, wrow, 0.0f, qc);
            sfq[f] = feature_value(p.map, d, f, sq, wrow, 0.0f, qc);
        }
    }
    __syncthreads();

    const int c4 = t % q4;
    const f32x4 vq = f32x4{sv[4 * c4], sv[4 * c4 + 1], sv[4 * c4 + 2], sv[4 * c4 + 3]};
    f32x4 acc = zero4();
#pragma unroll
    for (int i = 0; i < kDecHeld; i++) {
        const int e4 = t + kDecThreads * i;
        if (e4 < n4) {
            const int f = e4 / q4;
            f32x4 s = held[i];
            const float a = sfk[f];
            s[0] = fmaf(a, vq[0], s[0]);
            s[1] = fmaf(a, vq[1], s[1]);
            s[2] = fmaf(a, vq[2], s[2]);
            s[3] = fmaf(a, vq[3], s[3]);
            __builtin_nontemporal_store(s, S4 + e4);
            const float gq = sfq[f];
            acc[0] = fmaf(gq, s[0], acc[0]);
            acc[1] = fmaf(gq, s[1], acc[1]);
            acc[2] = fmaf(gq, s[2], acc[2]);
            acc[3] = fmaf(gq, s[3], acc[3]);
        }
    }
#pragma unroll 16
    for (int e4 = t + kDecThreads * kDecHeld; e4 < n4; e4 += kDecThreads) {
        const int f = e4 / q4;
        f32x4 s = __builtin_nontemporal_load(S4 + e4);
        const float a = sfk[f];
        s[0] = fmaf(a, vq[0], s[0]);
        s[1] = fmaf(a, vq[1], s[1]);
        s[2] = fmaf(a, vq[2], s[2]);
        s[3] = fmaf(a, vq[3], s[3]);
        __builtin_nontemporal_store(s, S4 + e4);
        const float gq = sfq[f];
        acc[0] = fmaf(gq, s[0], acc[0]);
        acc[1] = fmaf(gq, s[1], acc[1]);
        acc[2] = fmaf(gq, s[2], acc[2]);
        acc[3] = fmaf(gq, s[3], acc[3]);
    }
    float dpart = 0.0f;
    float *zb = p.z + (size_t)bh * dp;
    for (int f = t; f < dp; f += kDecThreads) {
        const float zz = zb[f] + sfk[f];
        zb[f] = zz;
        dpart = fmaf(sfq[f], zz, dpart);
    }
    sred[t] = acc;
    for (int o = 32; o > 0; o >>= 1) dpart += __shfl_xor(dpart, o);
    if ((t & 63) == 0) sden[t >> 6] = dpart;
    __syncthreads();
    if (t < q4) {
        f32x4 num = zero4();
        for (int u = t; u < kDecThreads; u += q4) num += sred[u];
        float den = 0.0f;
        for (int wv = 0; wv < kDecThreads / 64; wv++) den += sden[wv];
        for (int c = 0; c < 4; c++) st(p.y, (size_t)bh * d + 4 * t + c, num[c] / den, dt);
    }
}

// decode_kernel at compile-time sizes for the exponential maps with a bf16 W: the same loads and
// arithmetic with no load behind a branch.  At a branch's join the compiler no longer counts the
// outstanding loads and waits for all of them, so in decode_kernel the feature maps wait for the
// whole state; here they wait only for the token and W, which are requested first, and run while
// the state arrives (25.8 -> 24.9 us per step at B16 H32 d128).
template <int D, int DP>
__global__ __launch_bounds__(256) void decode_fixed_kernel(DecodeParams p) {
    constexpr int NT = 256, Q4 = D / 4, NP = DP * Q4 / NT;
    constexpr int TPR = NT / D, EPT = D / TPR, WP = EPT / 8;
    static_assert(DP * Q4 % NT == 0 && WP >= 1, "whole pieces per thread");
    __shared__ float sq[D], sk[D], sv[D];
    __shared__ float sfq[DP], sfk[DP];
    __shared__ f32x4 sred[NT];
    __shared__ float sden[NT / 64];
    const int bh = blockIdx.x, h = bh % p.H, t = threadIdx.x;
    const bf16_t *Wb = reinterpret_cast<const bf16_t *>(p.W);
    const int tc = t % D;
    const bf16_t xq = reinterpret_cast<const bf16_t *>(p.q)[(size_t)bh * D + tc];
    const bf16_t xk = reinterpret_cast<const bf16_t *>(p.k)[(size_t)bh * D + tc];
    const bf16_t xv = reinterpret_cast<const bf16_t *>(p.v)[(size_t)bh * D + tc];
    const int l = t / TPR, part = t % TPR;
    bf16x8 wreg[WP];
#pragma unroll
    for (int j = 0; j < WP; j++) wreg[j] = load8(Wb + ((size_t)h * D + l) * D + part * EPT + 8 * j);
    const bf16_t bb = *(p.b ? reinterpret_cast<const bf16_t *>(p.b) + (size_t)h * D + l : Wb);
    __builtin_amdgcn_sched_barrier(0);  // these requests leave before the state's
    f32x4 *S4 = reinterpret_cast<f32x4 *>(p.S + (size_t)bh * DP * D);
    f32x4 held[NP];
#pragma unroll
    for (int i = 0; i < NP; i++) held[i] = __builtin_nontemporal_load(S4 + t + NT * i);
    __builtin_amdgcn_sched_barrier(0);  // and the state's before anything waits for the token
    sq[tc] = bf16_bits_to_float(xq);
    sk[tc] = bf16_bits_to_float(xk);
    sv[tc] = bf16_bits_to_float(xv);
    __syncthreads();
    float uq = 0.0f, uk = 0.0f;
#pragma unroll
    for (int j = 0; j < WP; j++)
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const float wf = (float)wreg[j][e];
            uq = fmaf(wf, sq[part * EPT + 8 * j + e], uq);
            uk = fmaf(wf, sk[part * EPT + 8 * j + e], uk);
        }
#pragma unroll
    for (int o = TPR / 2; o > 0; o >>= 1) {
        uq += __shfl_xor(uq, o);
        uk += __shfl_xor(uk, o);
    }
    if (part == 0) {
        const float bl = p.b ? bf16_bits_to_float(bb) : 0.0f;
        sfq[l] = expf(uq + bl);
        sfk[l] = expf(uk + bl);
        if (DP == 2 * D) {
            sfq[D + l] = expf(-(uq + bl));
            sfk[D + l] = expf(-(uk + bl));
        }
    }
    __syncthreads();
    const int c4 = t % Q4;
    const f32x4 vq = f32x4{sv[4 * c4], sv[4 * c4 + 1], sv[4 * c4 + 2], sv[4 * c4 + 3]};
    // every piece of the state in before the first update: the updates and their stores then go
    // out in one burst (measured faster than updating each piece as it arrives)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    f32x4 acc = zero4();
#pragma unroll
    for (int i = 0; i < NP; i++) {
        const int f = (t + NT * i) / Q4;
        f32x4 x4 = held[i];
        const float a = sfk[f];
        x4[0] = fmaf(a, vq[0], x4[0]);
        x4[1] = fmaf(a, vq[1], x4[1]);
        x4[2] = fmaf(a, vq[2], x4[2]);
        x4[3] = fmaf(a, vq[3], x4[3]);
        __builtin_nontemporal_store(x4, S4 + t + NT * i);
        const float gq = sfq[f];
        acc[0] = fmaf(gq, x4[0], acc[0]);
        acc[1] = fmaf(gq, x4[1], acc[1]);
        acc[2] = fmaf(gq, x4[2], acc[2]);
        acc[3] = fmaf(gq, x4[3], acc[3]);
    }
    float dpart = 0.0f;
    float *zb = p.z + (size_t)bh * DP;
    if (t < DP) {
        const float zz = zb[t] + sfk[t];
        zb[t] = zz;
        dpart = sfq[t] * zz;
    }
    sred[t] = acc;
    for (int o = 32; o > 0; o >>= 1) dpart += __shfl_xor(dpart, o);
    if ((t & 63) == 0) sden[t >> 6] = dpart;
    __syncthreads();
    if (t < Q4) {
        f32x4 num = zero4();
        for (int u = t; u < NT; u += Q4) num += sred[u];
        float den = 0.0f;
        for (int w = 0; w < NT / 64; w++) den += sden[w];
        bf16_t *yb = reinterpret_cast<bf16_t *>(p.y) + (size_t)bh * D + 4 * t;
        for (int c = 0; c < 4; c++) yb[c] = float_to_bf16_bits(num[c] / den);
    }
}

hipError_t launch_decode(const DecodeParams &p, int BH, hipStream_t st) {
    const bool fixed = p.dtype == 1 && (p.map == HH_MAP_HEDGEHOG_ || p.map == HH_MAP_EXP_);
    if (fixed && p.d == 128 && p.dp == 256) hipLaunchKernelGGL((decode_fixed_kernel<128, 256>), dim3(BH), dim3(256), 0, st, p);
    else if (fixed && p.d == 128 && p.dp == 128) hipLaunchKernelGGL((decode_fixed_kernel<128, 128>), dim3(BH), dim3(256), 0, st, p);
    else if (fixed && p.d == 64 && p.dp == 128) hipLaunchKernelGGL((decode_fixed_kernel<64, 128>), dim3(BH), dim3(256), 0, st, p);
    else hipLaunchKernelGGL(decode_kernel, dim3(BH), dim3(kDecThreads), 0, st, p);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------------------
// Feature map on the vector units.  Hedgehog: one thread per (token, direction) writes
// both halves.  Taylor: one thread per (token, feature).
__global__ void fm_generic_kernel(int map, int dtype, int d, int dp, const void *x, const void *W, const void *b,
                                  void *phi, long ntok, int H, int N) {
    const long per = map == 0 ? d : dp;
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= ntok * per) return;
    const long tok = idx / per;
    const int f = (int)(idx % per);
    const size_t xo = (size_t)tok * d;
    if (map == 0) {
        const int h = (int)((tok / N) % H);
        const size_t wo = ((size_t)h * d + f) * d;
        float u = b ? ld(b, (size_t)h * d + f, dtype) : 0.0f;
        for (int m = 0; m < d; m++) u = fmaf(ld(W, wo + m, dtype), ld(x, xo + m, dtype), u);
        st(phi, (size_t)tok * dp + f, expf(u), dtype);
        st(phi, (size_t)tok * dp + d + f, expf(-u), dtype);
    } else {  // quadratic kernels; W: the generalised map's fp32 coefficients (null for Taylor)
        const QuadCoef qc = quad_coef(reinterpret_cast<const float *>(W), (int)((tok / N) % H));
        float val;
        if (f == 0) val = qc.sa;
        else if (f <= d) val = ld(x, xo + f - 1, dtype) * qc.sb;
        else {
            const int q = f - 1 - d;
            val = ld(x, xo + q / d, dtype) * ld(x, xo + q % d, dtype) * qc.sc;
        }
        st(phi, (size_t)tok * dp + f, val, dtype);
    }
}

hipError_t launch_featuremap_generic(int map, int dtype, int d, int dp, const void *x, const void *W, const void *b,
                                     void *phi, long BH, int H, int N, hipStream_t st) {
    const long ntok = BH * (long)N;
    const long per = map == 0 ? d : dp;
    const long total = ntok * per;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(fm_generic_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, map, dtype, d, dp,
                       x, W, b, phi, ntok, H, N);
    return hipGetLastError();
}

}  // namespace hh
