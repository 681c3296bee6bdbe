// svd_prep.hip -- SVDQuant weight preparation: W [N, K] -> bf16 low-rank pair
// (l2 [N, r], l1 [r, K]) plus the bf16 residual R = W - l2 . l1.
//
// OneTrainer PR #1034 "SVDQuant" / wiki SVDQuant entry: the weight is split
// into a bf16 low-rank part (rank 16-32) and a residual quantized like any
// W8A8 weight.  The low-rank part is the rank-r truncated SVD of W, stored
// balanced: l2 = U_r S_r^(1/2), l1 = S_r^(1/2) V_r^T.
//
// The truncated SVD is computed by randomized subspace iteration (Halko,
// Martinsson and Tropp, "Finding structure with randomness", SIAM Review 2011,
// randomized subspace iteration): with s = r + oversampling columns and a
// Gaussian test matrix Omega [s, K] supplied by the caller,
//   Q = orth(W Omega^T);  q times: Z = orth(W^T Q), Q = orth(W Z);
//   Zk = W^T Q  (so B = Q^T W = Zk^T);  B B^T = Zk^T Zk = U_B diag(lambda) U_B^T;
//   U = Q U_B,  V S = Zk U_B,  sigma = sqrt(lambda).
// orth() is Cholesky-QR applied twice (Gram matrix in f64).  The two large
// products read W once each (W^T is materialized once in the workspace); the
// s x s work (Cholesky, triangular inverse, Jacobi eigensolver) runs in f64
// in one workgroup.  Everything is on the GPU; the host only sequences
// launches.
#include "internal.hpp"

namespace w8a8 {
namespace {

constexpr int kMaxS = 64;
constexpr int kThreads = 256;
constexpr int kGramParts = 64;   // fixed: the reduction order does not depend on the device
typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- transpose
// out [cols, rows] = in [rows, cols]^T, bf16, 64 x 64 tiles through LDS.
__global__ __launch_bounds__(kThreads) void transpose_bf16_kernel(const uint16_t *__restrict__ in, int rows, int cols,
                                                                  uint16_t *__restrict__ out) {
    __shared__ uint16_t t[64][66];
    const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int i = ty; i < 64; i += 4) {
        const int r = r0 + i, c = c0 + tx;
        t[i][tx] = (r < rows && c < cols) ? in[(size_t)r * cols + c] : (uint16_t)0;
    }
    __syncthreads();
    for (int i = ty; i < 64; i += 4) {
        const int c = c0 + i, r = r0 + tx;
        if (c < cols && r < rows) out[(size_t)c * rows + r] = t[tx][i];
    }
}

// ---------------------------------------------------------------- thin product
// C[m, j] = sum_l A[m, l] (Bhi[j, l] + Blo[j, l]) for 16 rows per workgroup,
// j < sp (multiple of 16); A bf16 [rows, L], B bf16 [sp, L] (Blo may be
// null); C f32 [rows, sp].  L % 8 == 0.  Wave w takes the 32-wide l steps
// w, w + 4, ...; partial sums meet in LDS.
__global__ __launch_bounds__(kThreads) void thin_product_kernel(const uint16_t *__restrict__ a, int rows, int L,
                                                                const uint16_t *__restrict__ bhi,
                                                                const uint16_t *__restrict__ blo, int sp,
                                                                float *__restrict__ c) {
    __shared__ float part[4][16][kMaxS + 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m0 = blockIdx.x * 16;
    const int lq = (lane >> 4) * 8;
    const int nsteps = (L + 31) / 32;
    const int jb = sp / 16;
    v4f acc[kMaxS / 16];
#pragma unroll
    for (int b = 0; b < kMaxS / 16; ++b) acc[b] = v4f{0.f, 0.f, 0.f, 0.f};
    // Buffer ranges: this workgroup's rows of A, and B whole; rows past
    // `rows` and l past L read zero (out-of-range offsets), so the loads need
    // no branches and kU steps' loads are all in flight before their MFMAs.
    // (sizes stay below 0x7FFFFFF0: sp <= 64 and L < 2^24, checked on the host)
    const int rows_in = min(16, rows - m0);
    const int a_bytes = (int)((int64_t)rows_in * L * 2), b_bytes = (int)((int64_t)sp * L * 2);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a + (size_t)m0 * L), (short)0, a_bytes, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t rh =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(bhi), (short)0, b_bytes, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(blo ? blo : bhi), (short)0, blo ? b_bytes : 0, kBufferRsrcWord3);
    constexpr int kU = 4;  // steps per batch of loads
    constexpr int kOut = 0x7FFFFFF0;
    for (int st0 = wave; st0 < nsteps; st0 += 4 * kU) {
        v4u av[kU], h[kU][kMaxS / 16], lo[kU][kMaxS / 16];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int l = (st0 + 4 * u) * 32 + lq;
            const bool lin = l + 8 <= L;
            av[u] = __builtin_bit_cast(
                v4u, __builtin_amdgcn_raw_buffer_load_b128(ra, lin ? ((lane & 15) * L + l) * 2 : kOut, 0, 0));
#pragma unroll
            for (int b = 0; b < kMaxS / 16; ++b) {
                const int j = b * 16 + (lane & 15);
                const int off = lin && b < jb ? (j * L + l) * 2 : kOut;
                h[u][b] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rh, off, 0, 0));
                lo[u][b] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rl, off, 0, 0));
            }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const v8bf_t x = __builtin_bit_cast(v8bf_t, av[u]);
#pragma unroll
            for (int b = 0; b < kMaxS / 16; ++b) {
                if (b >= jb) break;
                acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, __builtin_bit_cast(v8bf_t, h[u][b]), acc[b], 0, 0, 0);
                if (blo)
                    acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, __builtin_bit_cast(v8bf_t, lo[u][b]), acc[b],
                                                                     0, 0, 0);
            }
        }
    }
    // 16x16 C layout: lane l, element i -> row 4(l / 16) + i, column l % 16
#pragma unroll
    for (int b = 0; b < kMaxS / 16; ++b) {
        if (b >= jb) break;
#pragma unroll
        for (int i = 0; i < 4; ++i) part[wave][4 * (lane >> 4) + i][b * 16 + (lane & 15)] = acc[b][i];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < 16 * sp; idx += kThreads) {
        const int rr = idx / sp, j = idx % sp;
        const int m = m0 + rr;
        if (m < rows) c[(size_t)m * sp + j] = part[0][rr][j] + part[1][rr][j] + part[2][rr][j] + part[3][rr][j];
    }
}

// ---------------------------------------------------------------- Gram partials
// partial[g][i][j] = sum over rows of chunk g of C[row, i] C[row, j] (f64),
// chunk g = rows [g * chunk, (g + 1) * chunk).  Thread t owns the bs x bs block
// of entries (bs = sp / 16) at block row t / 16, block column t % 16; a tile
// of 64 rows sits in LDS as f64, and each entry is summed over the tile's rows
// in order, then added to the entry's running sum (the products are exact in
// f64, one rounding per addition).
__global__ __launch_bounds__(kThreads) void gram_partial_kernel(const float *__restrict__ c, int rows, int sp,
                                                                int chunk, double *__restrict__ partial) {
    __shared__ double tile[64][kMaxS + 1];
    constexpr int kB = kMaxS / 16;  // largest block edge
    const int g = blockIdx.x, t = threadIdx.x;
    const int bs = sp / 16, i0 = (t / 16) * bs, j0 = (t % 16) * bs;
    const int r_begin = g * chunk, r_end = min(rows, r_begin + chunk);
    double acc[kB][kB];
#pragma unroll
    for (int a = 0; a < kB; ++a)
#pragma unroll
        for (int b = 0; b < kB; ++b) acc[a][b] = 0.0;
    for (int r0 = r_begin; r0 < r_end; r0 += 64) {
        const int nr = min(64, r_end - r0);
        __syncthreads();
        for (int idx = t; idx < 64 * sp; idx += kThreads) {
            const int rr = idx / sp, j = idx % sp;
            tile[rr][j] = rr < nr ? (double)c[(size_t)(r0 + rr) * sp + j] : 0.0;
        }
        __syncthreads();
        double s[kB][kB];
#pragma unroll
        for (int a = 0; a < kB; ++a)
#pragma unroll
            for (int b = 0; b < kB; ++b) s[a][b] = 0.0;
        for (int rr = 0; rr < nr; ++rr) {
            double xi[kB], xj[kB];
#pragma unroll
            for (int a = 0; a < kB; ++a) {
                xi[a] = a < bs ? tile[rr][i0 + a] : 0.0;
                xj[a] = a < bs ? tile[rr][j0 + a] : 0.0;
            }
#pragma unroll
            for (int a = 0; a < kB; ++a)
#pragma unroll
                for (int b = 0; b < kB; ++b) s[a][b] += xi[a] * xj[b];
        }
#pragma unroll
        for (int a = 0; a < kB; ++a)
#pragma unroll
            for (int b = 0; b < kB; ++b) acc[a][b] += s[a][b];
    }
#pragma unroll
    for (int a = 0; a < kB; ++a)
#pragma unroll
        for (int b = 0; b < kB; ++b)
            if (a < bs && b < bs) partial[(size_t)g * sp * sp + (size_t)(i0 + a) * sp + j0 + b] = acc[a][b];
}

// ---------------------------------------------------------------- s x s work
// One workgroup.  Sums the Gram partials in a fixed order, then
//  mode 0: G = R^T R (Cholesky, R upper); writes M = R^{-1} (f64 [sp, sp]).
//          A pivot at or below 1e-13 of the largest diagonal entry (a column
//          dependent on the previous ones) gets R[k][k] = 1 and a zero row, so
//          that column of the basis comes out (near) zero instead of blowing up.
//  mode 1: symmetric eigensolver (parallel cyclic Jacobi); writes M = the
//          eigenvectors (columns, eigenvalues descending), the singular values
//          sigma_j = sqrt(max(lambda_j, 0)) of the first r to `sigma`, and the
//          factor scales: fs[j] = sqrt(sigma_j) (l2) and fs[kMaxS + j] =
//          1 / sqrt(sigma_j) or 0 when sigma_j is negligible (l1).
__global__ __launch_bounds__(kThreads) void small_kernel(const double *__restrict__ partial, int sp, int mode, int r,
                                                         double *__restrict__ m_out, double *__restrict__ fs,
                                                         float *__restrict__ sigma) {
    __shared__ double A[kMaxS][kMaxS + 1];
    __shared__ double V[kMaxS][kMaxS + 1];
    __shared__ double rc[kMaxS / 2], rs[kMaxS / 2];
    __shared__ int pp[kMaxS / 2], pq[kMaxS / 2];
    __shared__ double red[kThreads];
    __shared__ int flag;
    const int t = threadIdx.x;
    for (int e = t; e < sp * sp; e += kThreads) {
        // all partials of the entry in flight at once, then summed in order
        double v[kGramParts];
#pragma unroll
        for (int g = 0; g < kGramParts; ++g) v[g] = partial[(size_t)g * sp * sp + e];
        double s = 0.0;
#pragma unroll
        for (int g = 0; g < kGramParts; ++g) s += v[g];
        A[e / sp][e % sp] = s;
    }
    __syncthreads();
    if (mode == 0) {
        double dmax = 0.0;
        for (int k = 0; k < sp; ++k) dmax = fmax(dmax, A[k][k]);
        const double tiny = 1e-13 * dmax;
        // Cholesky, right-looking (V holds R, upper): step k takes the pivot,
        // scales row k, then the whole workgroup subtracts the outer product
        // of row k from the trailing upper triangle of A -- the same products
        // subtracted in the same order (i ascending) as a column-by-column
        // formulation, spread over the threads instead of one dot product
        // per column.
        for (int e = t; e < sp * sp; e += kThreads) V[e / sp][e % sp] = 0.0;
        __syncthreads();
        for (int k = 0; k < sp; ++k) {
            if (t == 0) {
                const double d = A[k][k];
                flag = d > tiny && d > 0.0;
                V[k][k] = flag ? sqrt(d) : 1.0;
            }
            __syncthreads();
            for (int j = k + 1 + t; j < sp; j += kThreads) V[k][j] = flag ? A[k][j] / V[k][k] : 0.0;
            __syncthreads();
            const int n = sp - 1 - k;  // trailing size
            for (int e = t; e < n * n; e += kThreads) {
                const int i = k + 1 + e / n, j = k + 1 + e % n;
                if (i <= j) A[i][j] -= V[k][i] * V[k][j];
            }
            __syncthreads();
        }
        // X = R^{-1} (upper), one column per thread
        if (t < sp) {
            const int j = t;
            for (int i = 0; i < sp; ++i) A[i][j] = 0.0;
            A[j][j] = 1.0 / V[j][j];
            for (int i = j - 1; i >= 0; --i) {
                double s = 0.0;
                for (int k = i + 1; k <= j; ++k) s += V[i][k] * A[k][j];
                A[i][j] = -s / V[i][i];
            }
        }
        __syncthreads();
        for (int e = t; e < sp * sp; e += kThreads) m_out[e] = A[e / sp][e % sp];
        return;
    }
    // ---- mode 1: Jacobi.  V = I.
    for (int e = t; e < sp * sp; e += kThreads) V[e / sp][e % sp] = (e / sp == e % sp) ? 1.0 : 0.0;
    __syncthreads();
    const int np = sp / 2;  // sp is even (a multiple of 16)
    for (int sweep = 0; sweep < 40; ++sweep) {
        // convergence: largest off-diagonal magnitude vs the largest diagonal one
        double off = 0.0, dia = 0.0;
        for (int e = t; e < sp * sp; e += kThreads) {
            const int i = e / sp, j = e % sp;
            if (i == j) dia = fmax(dia, fabs(A[i][j]));
            else off = fmax(off, fabs(A[i][j]));
        }
        red[t] = off;
        __syncthreads();
        if (t == 0) {
            double o = 0.0;
            for (int i = 0; i < kThreads; ++i) o = fmax(o, red[i]);
            red[0] = o;
        }
        __syncthreads();
        const double offmax = red[0];
        __syncthreads();
        red[t] = dia;
        __syncthreads();
        if (t == 0) {
            double d = 0.0;
            for (int i = 0; i < kThreads; ++i) d = fmax(d, red[i]);
            flag = !(offmax > 1e-15 * d && offmax > 0.0);
        }
        __syncthreads();
        if (flag) break;
        // round-robin tournament: np pairs per step, sp - 1 steps per sweep
        for (int step = 0; step < sp - 1; ++step) {
            if (t < np) {
                // positions 0..sp-1 around a circle with 0 fixed; pair k: (k, sp-1-k)
                auto who = [&](int pos) { return pos == 0 ? 0 : 1 + (pos - 1 + step) % (sp - 1); };
                int p = who(t), q = who(sp - 1 - t);
                if (p > q) { const int x = p; p = q; q = x; }
                const double apq = A[p][q];
                double c = 1.0, s = 0.0;
                if (apq != 0.0) {
                    const double zeta = (A[q][q] - A[p][p]) / (2.0 * apq);
                    const double tt = (zeta >= 0.0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
                    c = 1.0 / sqrt(1.0 + tt * tt);
                    s = tt * c;
                }
                pp[t] = p; pq[t] = q; rc[t] = c; rs[t] = s;
            }
            __syncthreads();
            // A <- J^T A J one 2x2 block at a time: rows p, q of pair k and
            // columns p', q' of pair l, first rotated as rows by pair k, then
            // as columns by pair l (the pairs partition the indices, so the
            // blocks are disjoint); and V <- V J
            for (int e = t; e < np * np; e += kThreads) {
                const int k = e / np, l = e % np;
                const int p = pp[k], q = pq[k], p2 = pp[l], q2 = pq[l];
                const double c = rc[k], s = rs[k], c2 = rc[l], s2 = rs[l];
                const double apr = A[p][p2], aqr = A[q][p2], aps = A[p][q2], aqs = A[q][q2];
                const double bpr = c * apr - s * aqr, bqr = s * apr + c * aqr;
                const double bps = c * aps - s * aqs, bqs = s * aps + c * aqs;
                A[p][p2] = c2 * bpr - s2 * bps;
                A[p][q2] = s2 * bpr + c2 * bps;
                A[q][p2] = c2 * bqr - s2 * bqs;
                A[q][q2] = s2 * bqr + c2 * bqs;
            }
            for (int e = t; e < np * sp; e += kThreads) {
                const int k = e / sp, row = e % sp;
                const int p = pp[k], q = pq[k];
                const double c = rc[k], s = rs[k];
                const double vp = V[row][p], vq = V[row][q];
                V[row][p] = c * vp - s * vq;
                V[row][q] = s * vp + c * vq;
            }
            __syncthreads();
        }
    }
    // order by eigenvalue, descending (one thread; sp <= 64)
    __shared__ int order[kMaxS];
    if (t == 0) {
        for (int i = 0; i < sp; ++i) order[i] = i;
        for (int i = 0; i < sp; ++i) {
            int best = i;
            for (int j = i + 1; j < sp; ++j)
                if (A[order[j]][order[j]] > A[order[best]][order[best]]) best = j;
            const int x = order[i]; order[i] = order[best]; order[best] = x;
        }
    }
    __syncthreads();
    for (int e = t; e < sp * sp; e += kThreads) {
        const int i = e / sp, j = e % sp;
        m_out[e] = V[i][order[j]];
    }
    if (t < sp) {
        const double lam = A[order[t]][order[t]];
        const double sg = sqrt(fmax(lam, 0.0));
        double lam0 = fmax(A[order[0]][order[0]], 0.0);
        const bool live = sg > 1e-7 * sqrt(lam0) && sg > 0.0;
        fs[t] = live ? sqrt(sg) : 0.0;
        fs[kMaxS + t] = live ? 1.0 / sqrt(sg) : 0.0;
        if (t < r) sigma[t] = (float)sg;
    }
}

// ---------------------------------------------------------------- row x small
// out[row, j] = sum_i C[row, i] M[i][j] for 64 rows per workgroup.
//  mode 0 (basis): C is overwritten with the result (f32 [rows, sp]); when
//          thi is set, its bf16 hi/lo halves are written transposed,
//          thi/tlo [sp, rows].
//  mode 1 (factor, row-major): bf16 out [rows, r] = result * scale[j].
//  mode 2 (factor, transposed): bf16 out [r, rows] = result * scale[j].
__global__ __launch_bounds__(kThreads) void apply_small_kernel(float *__restrict__ c, int rows, int sp,
                                                               const double *__restrict__ m, int mode, int r,
                                                               const double *__restrict__ scale,
                                                               uint16_t *__restrict__ thi, uint16_t *__restrict__ tlo,
                                                               uint16_t *__restrict__ out) {
    __shared__ float ms[kMaxS][kMaxS + 1];
    __shared__ float cs[64][kMaxS + 1];
    const int r0 = blockIdx.x * 64;
    const int nr = min(64, rows - r0);
    for (int e = threadIdx.x; e < sp * sp; e += kThreads) ms[e / sp][e % sp] = (float)m[e];
    for (int e = threadIdx.x; e < 64 * sp; e += kThreads) {
        const int rr = e / sp, j = e % sp;
        cs[rr][j] = rr < nr ? c[(size_t)(r0 + rr) * sp + j] : 0.0f;
    }
    __syncthreads();
    const int ncol = mode == 0 ? sp : r;
    // thread -> (row rr = e % 64, column j = e / 64): consecutive threads take
    // consecutive rows, so the transposed writes are coalesced
    for (int e = threadIdx.x; e < 64 * ncol; e += kThreads) {
        const int rr = e % 64, j = e / 64;
        if (rr >= nr) continue;
        float v = 0.0f;
        for (int i = 0; i < sp; ++i) v = __builtin_fmaf(cs[rr][i], ms[i][j], v);
        const int row = r0 + rr;
        if (mode == 0) {
            c[(size_t)row * sp + j] = v;
            if (thi) {
                const uint32_t hi = f32_to_bf16_bits(v);
                thi[(size_t)j * rows + row] = (uint16_t)hi;
                tlo[(size_t)j * rows + row] = (uint16_t)f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
            }
        } else {
            const uint16_t b = (uint16_t)f32_to_bf16_bits((float)((double)v * scale[j]));
            if (mode == 1) out[(size_t)row * r + j] = b;
            else out[(size_t)j * rows + row] = b;
        }
    }
}

// ---------------------------------------------------------------- residual
// res[n, k] = bf16(W[n, k] - sum_j l2[n, j] l1[j, k]); 64 x 64 tiles, each
// thread a 4 x 4 block; products of bf16 values are exact in f32.
__global__ __launch_bounds__(kThreads) void residual_kernel(const uint16_t *__restrict__ w, int N, int K,
                                                            const uint16_t *__restrict__ l2,
                                                            const uint16_t *__restrict__ l1, int r,
                                                            uint16_t *__restrict__ res) {
    __shared__ float a[64][kMaxS + 1];  // l2 rows of the tile
    __shared__ float b[kMaxS][64 + 4];  // l1 columns of the tile
    const int n0 = blockIdx.y * 64, k0 = blockIdx.x * 64;
    for (int e = threadIdx.x; e < 64 * r; e += kThreads) {
        const int rr = e / r, j = e % r;
        a[rr][j] = n0 + rr < N ? bf16_bits_to_f32(l2[(size_t)(n0 + rr) * r + j]) : 0.0f;
    }
    for (int e = threadIdx.x; e < r * 64; e += kThreads) {
        const int j = e / 64, cc = e % 64;
        b[j][cc] = k0 + cc < K ? bf16_bits_to_f32(l1[(size_t)j * K + k0 + cc]) : 0.0f;
    }
    __syncthreads();
    const int tr = (threadIdx.x >> 4) * 4, tc = (threadIdx.x & 15) * 4;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][q] = 0.0f;
    for (int j = 0; j < r; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[i][q] = __builtin_fmaf(a[tr + i][j], b[j][tc + q], acc[i][q]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int n = n0 + tr + i;
        if (n >= N) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int k = k0 + tc + q;
            if (k < K) {
                const size_t o = (size_t)n * K + k;
                res[o] = (uint16_t)f32_to_bf16_bits(bf16_bits_to_f32(w[o]) - acc[i][q]);
            }
        }
    }
}

inline int64_t subspace(int64_t r) {
    const int64_t s = (r + 16 + 15) / 16 * 16;
    return s < kMaxS ? s : kMaxS;
}

struct Ws {
    uint16_t *wt;             // [K, N]
    float *cn, *ck;           // [N, s], [K, s]
    uint16_t *qhi, *qlo;      // [s, N]
    uint16_t *zhi, *zlo;      // [s, K]
    double *part;             // [kGramParts, s, s]
    double *m;                // [s, s]
    double *fs;               // [2 * kMaxS]
};

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Byte offsets of the workspace parts (one layout for the size query and the call).
inline size_t carve(int64_t N, int64_t K, int64_t s, uint8_t *base, Ws *ws) {
    size_t off = 0;
    auto take = [&](size_t bytes) -> uint8_t * {
        uint8_t *p = base ? base + off : nullptr;
        off += align256(bytes);
        return p;
    };
    Ws w;
    w.wt = reinterpret_cast<uint16_t *>(take((size_t)N * K * 2));
    w.cn = reinterpret_cast<float *>(take((size_t)N * s * 4));
    w.ck = reinterpret_cast<float *>(take((size_t)K * s * 4));
    w.qhi = reinterpret_cast<uint16_t *>(take((size_t)s * N * 2));
    w.qlo = reinterpret_cast<uint16_t *>(take((size_t)s * N * 2));
    w.zhi = reinterpret_cast<uint16_t *>(take((size_t)s * K * 2));
    w.zlo = reinterpret_cast<uint16_t *>(take((size_t)s * K * 2));
    w.part = reinterpret_cast<double *>(take((size_t)kGramParts * s * s * 8));
    w.m = reinterpret_cast<double *>(take((size_t)s * s * 8));
    w.fs = reinterpret_cast<double *>(take((size_t)2 * kMaxS * 8));
    if (ws) *ws = w;
    return off;
}

}  // namespace
}  // namespace w8a8

extern "C" int64_t svdq_prepare_subspace(int64_t r) {
    if (r < 1 || r > w8a8::kMaxS) return 0;
    return w8a8::subspace(r);
}

extern "C" size_t svdq_prepare_workspace_bytes(int64_t N, int64_t K, int64_t r) {
    if (N < 1 || K < 1 || r < 1 || r > w8a8::kMaxS) return 0;
    return w8a8::carve(N, K, w8a8::subspace(r), nullptr, nullptr);
}

extern "C" w8a8_status svdq_prepare(const uint16_t *w, int64_t N, int64_t K, int64_t r, const uint16_t *omega,
                                    int iters, uint16_t *l1, uint16_t *l2, uint16_t *residual, float *sigma,
                                    void *workspace, hipStream_t stream) {
    using namespace w8a8;
    if (N < 1 || K < 1 || r < 1 || r > kMaxS || iters < 0 || iters > 16) return W8A8_ERR_INVALID_ARG;
    if (r > N || r > K) return W8A8_ERR_SHAPE;
    if (N % 8 != 0 || K % 8 != 0 || N >= (1 << 24) || K >= (1 << 24) || N * K > ((int64_t)1 << 31))
        return W8A8_ERR_SHAPE;
    if (!w || !omega || !l1 || !l2 || !residual || !sigma || !workspace) return W8A8_ERR_INVALID_ARG;
    if (!aligned16(w) || !aligned16(omega) || !aligned16(l1) || !aligned16(l2) || !aligned16(residual) ||
        !aligned16(sigma) || !aligned16(workspace))
        return W8A8_ERR_ALIGN;
    const int s = (int)subspace(r);
    const int n = (int)N, k = (int)K, rr = (int)r;
    Ws ws;
    carve(N, K, s, static_cast<uint8_t *>(workspace), &ws);

    auto product = [&](const uint16_t *a, int rows, int L, const uint16_t *bhi, const uint16_t *blo, float *c) {
        thin_product_kernel<<<(rows + 15) / 16, kThreads, 0, stream>>>(a, rows, L, bhi, blo, s, c);
    };
    auto gram = [&](const float *c, int rows) {
        const int chunk = (rows + kGramParts - 1) / kGramParts;
        gram_partial_kernel<<<kGramParts, kThreads, 0, stream>>>(c, rows, s, chunk, ws.part);
    };
    // Cholesky-QR twice; the last pass also writes the transposed hi/lo copy
    auto orth = [&](float *c, int rows, uint16_t *thi, uint16_t *tlo) {
        for (int pass = 0; pass < 2; ++pass) {
            gram(c, rows);
            small_kernel<<<1, kThreads, 0, stream>>>(ws.part, s, 0, rr, ws.m, ws.fs, sigma);
            apply_small_kernel<<<(rows + 63) / 64, kThreads, 0, stream>>>(
                c, rows, s, ws.m, 0, rr, nullptr, pass == 1 ? thi : nullptr, pass == 1 ? tlo : nullptr, nullptr);
        }
    };

    transpose_bf16_kernel<<<dim3((k + 63) / 64, (n + 63) / 64), kThreads, 0, stream>>>(w, n, k, ws.wt);
    product(w, n, k, omega, nullptr, ws.cn);                  // Y = W Omega^T
    orth(ws.cn, n, ws.qhi, ws.qlo);                           // Q
    for (int it = 0; it < iters; ++it) {
        product(ws.wt, k, n, ws.qhi, ws.qlo, ws.ck);          // W^T Q
        orth(ws.ck, k, ws.zhi, ws.zlo);                       // Z
        product(w, n, k, ws.zhi, ws.zlo, ws.cn);              // W Z
        orth(ws.cn, n, ws.qhi, ws.qlo);                       // Q
    }
    product(ws.wt, k, n, ws.qhi, ws.qlo, ws.ck);              // Zk = W^T Q = B^T
    gram(ws.ck, k);                                           // B B^T
    small_kernel<<<1, kThreads, 0, stream>>>(ws.part, s, 1, rr, ws.m, ws.fs, sigma);
    // l2 = Q U_B S^(1/2), l1 = S^(-1/2) U_B^T Zk^T (= S^(1/2) V^T)
    apply_small_kernel<<<(n + 63) / 64, kThreads, 0, stream>>>(ws.cn, n, s, ws.m, 1, rr, ws.fs, nullptr, nullptr,
                                                                l2);
    apply_small_kernel<<<(k + 63) / 64, kThreads, 0, stream>>>(ws.ck, k, s, ws.m, 2, rr, ws.fs + kMaxS, nullptr,
                                                                nullptr, l1);
    residual_kernel<<<dim3((k + 63) / 64, (n + 63) / 64), kThreads, 0, stream>>>(w, n, k, l2, l1, rr, residual);
    return launch_status();
}
