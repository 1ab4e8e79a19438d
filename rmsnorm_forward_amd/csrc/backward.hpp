// backward.hpp -- LayerNorm / RMSNorm backward ("CUDA 算子工程" ch. 7,
// section 7.7), from the mean and rstd the forward pass stored.
//
// norm_bwd_rows_kernel: a team of TEAM lanes owns a row, as in the forward
// row kernel (lane t holds vectors j*TEAM + t).  Per row it reads dy and x
// once, forms xhat = (x - mean) * rstd and g = dy * gamma, reduces the two
// row sums the section names -- sum(g) and sum(g * xhat) for LayerNorm,
// sum(g * x) for RMSNorm -- in one exchange, and writes
//   LayerNorm  dx = rstd * (g - mean(g) - xhat * mean(g xhat))
//   RMSNorm    dx = rstd * g - x * rstd^3 * mean(g x)
// The column sums dgamma = sum_rows dy * xhat (RMSNorm: dy * x * rstd) and
// dbeta = sum_rows dy are accumulated in fp32 registers by the lane that
// owns each column, over the rows its team visits (a fixed grid, row groups
// grid-strided), summed over the workgroup's teams and written as one
// partial row per workgroup: part_* is [gridDim.x, N].
//
// The grid is persistent (about one workgroup per CU), so each team walks many
// rows one after another; where registers allow, the next row's dy, x and
// statistics are loaded while the current row is reduced and written.
// gamma -- the same columns for every row a lane sees -- is loaded once.
//
// norm_colsum_kernel: sums the partial rows of each column in a fixed order,
// so dgamma and dbeta are bitwise reproducible for a given grid.
#pragma once

#include "dispatch.hpp"
#include "prims.hpp"
#include "rows.hpp"

namespace mi355norm {

// Backward workgroups hold kBwdWG lanes, i.e. kBwdWG / TEAM rows at once.
template <int TEAM>
struct BwdGeom {
    static constexpr int WG = kBwdWG;
    static constexpr int ROWS = WG / TEAM;                 // rows per workgroup
    static constexpr int WPT = TEAM > 64 ? TEAM / 64 : 1;  // wavefronts per team
};

template <class T, bool RMS, int TEAM, int VPL, int EPV>
__global__ __launch_bounds__(kBwdWG)
void norm_bwd_rows_kernel(const typename T::storage* dy,      // dx may be written over dy or x
                          const typename T::storage* x,
                          const typename T::storage* __restrict__ gamma,
                          const float* __restrict__ mean,
                          const float* __restrict__ rstd,
                          typename T::storage* dx,
                          float* __restrict__ part_g,      // [gridDim.x, N] partial dgamma rows (or null)
                          float* __restrict__ part_b,      // [gridDim.x, N] partial dbeta rows (or null)
                          int64_t M, int N, int64_t ldy, int64_t ldx, int64_t lddx)
{
    using G = BwdGeom<TEAM>;
    using S = typename T::storage;
    using V = Vec<T, EPV>;
    __shared__ float2 red[2][G::ROWS][G::WPT];

    const int tid = threadIdx.x;
    const int team = TEAM >= 64 ? __builtin_amdgcn_readfirstlane(tid / TEAM) : tid / TEAM;
    const int tl = tid % TEAM;
    const int wave_in_team = TEAM > 64 ? __builtin_amdgcn_readfirstlane(tl >> 6) : 0;
    const int NV = N / EPV;
    const float inv_n = 1.0f / (float)N;
    const bool want_g = part_g != nullptr;
    const bool want_b = part_b != nullptr;

    bool col_ok[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) col_ok[j] = (int)(j * TEAM + tl) < NV;

    // Column accumulators.  LayerNorm keeps two per element; with more than
    // 16 elements per lane (8 on the element-wise path, where each element
    // takes a VGPR) the registers run out (a 1024-lane workgroup may hold 128
    // VGPRs), so its dbeta accumulators live in LDS instead: [element][lane],
    // 128 KiB at 32 elements, consecutive lanes at consecutive addresses;
    // each lane touches only its own slots.  gamma is then re-read (from the
    // caches) for every row instead of held.  Measured, bf16 4096 x 32768:
    // LayerNorm 316 -> 212 us; the same for RMSNorm's single accumulator was
    // slower (154 -> 170 us), so RMSNorm keeps it in registers.
    constexpr int E = VPL * EPV;
    constexpr bool LACC = !RMS && (E > 16 || (EPV == 1 && E > 8));
    // With at most 8 elements per lane, g and xhat (RMSNorm: x) stay in fp32
    // registers across the exchange and the column sums are taken in the
    // first pass, so the second pass only forms dx (LN bf16 16384 x 8192:
    // 148.8 -> 147.9 us, 65536 x 2048: 137.6 -> 135.8; at 16 elements per
    // lane the copies spill: 167 -> 184 us).  Longer lanes re-widen dy and x.
    constexpr bool KEEP = !LACC && E <= 8;

    // gamma of this lane's columns (ones without gamma), kept packed for
    // every row
    V gam[LACC ? 1 : VPL];
    auto gamma_vec = [&](int j) {
        V g;
        if (gamma != nullptr && col_ok[j]) {
            g.load(gamma + (j * TEAM + tl) * EPV);
        } else {
            float one[EPV];
#pragma unroll
            for (int k = 0; k < EPV; ++k) one[k] = 1.0f;
            g.set(one);
        }
        return g;
    };
    if constexpr (!LACC) {
#pragma unroll
        for (int j = 0; j < VPL; ++j) gam[j] = gamma_vec(j);
    }
    auto gam_at = [&](int j) {
        if constexpr (LACC) return gamma_vec(j);
        else return gam[j];
    };

    // with 16-byte vectors a lane's four consecutive columns share one LDS
    // slot ([column / 4][lane], float4), else [column][lane]
    constexpr bool LACC4 = LACC && EPV % 4 == 0;
    __shared__ float acc_lds[LACC && !LACC4 ? E : 1][kBwdWG];
    __shared__ float4 acc_lds4[LACC4 ? E / 4 : 1][kBwdWG];
    float acc_g[VPL][EPV], acc_b[(RMS || LACC) ? 1 : VPL][EPV];
#pragma unroll
    for (int j = 0; j < VPL; ++j)
#pragma unroll
        for (int k = 0; k < EPV; ++k) {
            acc_g[j][k] = 0.0f;
            if constexpr (!RMS && !LACC) acc_b[j][k] = 0.0f;
            if constexpr (LACC && !LACC4) acc_lds[j * EPV + k][tid] = 0.0f;
            if constexpr (LACC4)
                if (k % 4 == 0) acc_lds4[(j * EPV + k) / 4][tid] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }

    // the loads of one row group: dy, x and the row's statistics
    const int64_t groups = (M + G::ROWS - 1) / G::ROWS;
    auto fetch = [&](int64_t grp, V (&d)[VPL], V (&xx)[VPL], float& m, float& r) {
        const int64_t row = grp * G::ROWS + team;
        const bool row_ok = grp < groups && row < M;
        const int64_t rr = row_ok ? row : 0;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const unsigned v = (unsigned)(j * TEAM + tl);
            if (row_ok && col_ok[j]) {
                d[j].load_stream(dy + rr * ldy + v * EPV);
                xx[j].load_stream(x + rr * ldx + v * EPV);
            }
        }
        m = (!RMS && row_ok) ? mean[rr] : 0.0f;
        r = row_ok ? rstd[rr] : 0.0f;
    };
    // One row group: the two row sums, dx, and the column accumulators.
    // d, xx, m, r hold the group's loads; par picks the LDS exchange slots
    // (consecutive groups alternate, so one barrier per group suffices).
    // before_stores runs once dx is computed (d and xx are dead then),
    // before dx is stored.
    auto row_group = [&](int64_t grp, V (&d)[VPL], V (&xx)[VPL], float m, float r, int par,
                         auto&& before_stores) {
        const int64_t row = grp * G::ROWS + team;
        const bool row_ok = row < M;
        const int64_t rr = row_ok ? row : 0;
        bool ok[VPL];
#pragma unroll
        for (int j = 0; j < VPL; ++j) ok[j] = row_ok && col_ok[j];

        // the row sums: (sum g, sum g xhat) for LayerNorm, (0, sum g x) for RMSNorm
        float s1 = 0.0f, s2 = 0.0f;
        float gk[KEEP ? VPL : 1][KEEP ? EPV : 1], hk[KEEP ? VPL : 1][KEEP ? EPV : 1];
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            if (!ok[j]) continue;
            const V gj = gam_at(j);
#pragma unroll
            for (int k = 0; k < EPV; ++k) {
                const float dk = d[j].get(k);
                const float g = dk * gj.get(k);
                const float xh = RMS ? xx[j].get(k) : (xx[j].get(k) - m) * r;
                if constexpr (!RMS) s1 += g;
                s2 = __builtin_fmaf(g, xh, s2);
                if constexpr (KEEP) {
                    gk[j][k] = g;
                    hk[j][k] = xh;
                    if constexpr (RMS) {
                        acc_g[j][k] = __builtin_fmaf(dk, xh * r, acc_g[j][k]);
                    } else {
                        acc_g[j][k] = __builtin_fmaf(dk, xh, acc_g[j][k]);
                        acc_b[j][k] += dk;
                    }
                }
            }
        }
        if constexpr (!KEEP) {
            // re-widen dy and x after the exchange rather than keep fp32
            // copies live across it
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                d[j].opaque();
                xx[j].opaque();
            }
        }
        if constexpr (!RMS) s1 = team_sum<(TEAM < 64 ? TEAM : 64)>(s1);
        s2 = team_sum<(TEAM < 64 ? TEAM : 64)>(s2);
        if constexpr (TEAM > 64) {
            if (lane_id() == 0) red[par][team][wave_in_team] = make_float2(s1, s2);
            __syncthreads();
            float a = 0.0f, b = 0.0f;
#pragma unroll
            for (int w = 0; w < G::WPT; ++w) {
                a += red[par][team][w].x;
                b += red[par][team][w].y;
            }
            s1 = a;
            s2 = b;
        }
        // LayerNorm: dx = r (g - c1 - xhat c2); RMSNorm: dx = r g - x c2
        const float c1 = s1 * inv_n;
        const float c2 = RMS ? r * r * r * (s2 * inv_n) : s2 * inv_n;
        S* dxr = dx + rr * lddx;
        V out[VPL];
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            if (!ok[j]) continue;
            const V gj = gam_at(j);
            float o[EPV];
#pragma unroll
            for (int k = 0; k < EPV; ++k) {
                if constexpr (KEEP) {
                    if constexpr (RMS) o[k] = __builtin_fmaf(r, gk[j][k], -hk[j][k] * c2);
                    else o[k] = r * ((gk[j][k] - c1) - hk[j][k] * c2);
                    continue;
                }
                const float dk = d[j].get(k);
                const float g = dk * gj.get(k);
                if constexpr (RMS) {
                    const float xk = xx[j].get(k);
                    o[k] = __builtin_fmaf(r, g, -xk * c2);
                    acc_g[j][k] = __builtin_fmaf(dk, xk * r, acc_g[j][k]);
                } else {
                    const float xh = (xx[j].get(k) - m) * r;
                    o[k] = r * ((g - c1) - xh * c2);
                    acc_g[j][k] = __builtin_fmaf(dk, xh, acc_g[j][k]);
                    if constexpr (LACC && !LACC4) acc_lds[j * EPV + k][tid] += dk;
                    else if constexpr (!LACC) acc_b[j][k] += dk;
                }
            }
            if constexpr (LACC4) {
#pragma unroll
                for (int q = 0; q < EPV / 4; ++q) {
                    float4 a = acc_lds4[j * (EPV / 4) + q][tid];
                    a.x += d[j].get(4 * q);
                    a.y += d[j].get(4 * q + 1);
                    a.z += d[j].get(4 * q + 2);
                    a.w += d[j].get(4 * q + 3);
                    acc_lds4[j * (EPV / 4) + q][tid] = a;
                }
            }
            out[j].set(o);           // rounded to the storage type (RNE)
        }
        before_stores();
#pragma unroll
        for (int j = 0; j < VPL; ++j)
            if (ok[j]) out[j].put_stream(dxr + (unsigned)(j * TEAM + tl) * EPV);
    };

    // The next row group's loads are issued before this one is worked on
    // when the registers allow: LIVE counts the VGPRs held across rows (dy,
    // x, gamma, the column accumulators), and a second copy of dy and x must
    // keep the total well under the 128 a 1024-lane workgroup may use.  The
    // loop is unrolled by two over register sets A and B, so that no copy
    // between them forces an early wait.  Loads and stores share one
    // completion counter and may complete out of order with respect to each
    // other, so a wait for loads issued before a store is a wait for the
    // store too; each row therefore waits for the next row's loads (which
    // have been in flight during its work) before it issues its own stores.
    constexpr int WORDS = (EPV * (int)sizeof(S) + 3) / 4;   // VGPRs per vector
    constexpr int LIVE = (LACC ? 2 : 3) * VPL * WORDS + ((RMS ? 1 : 2) - (LACC ? 1 : 0)) * VPL * EPV;
    constexpr bool PREFETCH = LIVE + 2 * VPL * WORDS <= 80;
    const int64_t stride = gridDim.x;
    V dA[VPL], xA[VPL];
    float mA, rA;
    fetch(blockIdx.x, dA, xA, mA, rA);
    if constexpr (PREFETCH) {
        V dB[VPL], xB[VPL];
        float mB, rB;
        auto ready = [&](V (&d)[VPL], V (&xx)[VPL], float& m, float& r) {
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                d[j].opaque();
                xx[j].opaque();
            }
            asm volatile("" : "+v"(m), "+v"(r));
        };
        // (ready() runs on every path, the first group's loads included: a
        // load still pending where paths join makes its first use wait
        // again, for everything issued since)
        ready(dA, xA, mA, rA);
        for (int64_t grp = blockIdx.x; grp < groups;) {
            fetch(grp + stride, dB, xB, mB, rB);
            row_group(grp, dA, xA, mA, rA, 0, [&] { ready(dB, xB, mB, rB); });
            grp += stride;
            if (grp >= groups) break;
            fetch(grp + stride, dA, xA, mA, rA);
            row_group(grp, dB, xB, mB, rB, 1, [&] { ready(dA, xA, mA, rA); });
            grp += stride;
        }
    } else {
        // one register set: the next group's loads go into it once this
        // group's dx is computed, before its stores (measured, bf16
        // 4096 x 32768: LayerNorm 222 -> 215 us, RMSNorm 156 -> 150 us)
        int par = 0;
        for (int64_t grp = blockIdx.x; grp < groups; grp += stride, par ^= 1)
            row_group(grp, dA, xA, mA, rA, par, [&] { fetch(grp + stride, dA, xA, mA, rA); });
    }

    // One partial row per workgroup.  Teams own the same columns lane for
    // lane (lane tl of every team holds vectors j*TEAM + tl), so with several
    // teams per workgroup team 0 adds the others' accumulators, one element
    // at a time through LDS, in team order.
    __shared__ float xch[G::ROWS > 1 ? G::WG : 1];
    auto fold = [&](float& a) {
        __syncthreads();
        xch[tid] = a;
        __syncthreads();
        if (team == 0) {
            float t = xch[tl];
#pragma unroll
            for (int q = 1; q < G::ROWS; ++q) t += xch[q * TEAM + tl];
            a = t;
        }
    };
    const int64_t prow = blockIdx.x;
    // a lane's EPV consecutive columns go out as 16-byte vectors where EPV
    // allows (the partial rows are 16-byte aligned then)
    auto put_row = [&](float* dst, const float (&v)[EPV]) {
        if constexpr (EPV % 4 == 0) {
#pragma unroll
            for (int k = 0; k < EPV; k += 4)
                *reinterpret_cast<float4*>(dst + k) = make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]);
        } else {
#pragma unroll
            for (int k = 0; k < EPV; ++k) dst[k] = v[k];
        }
    };
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        const unsigned off = (unsigned)(j * TEAM + tl) * EPV;
        float vg[EPV], vb[EPV];
#pragma unroll
        for (int k = 0; k < EPV; ++k) {
            float ag = acc_g[j][k], ab = 0.0f;
            if constexpr (LACC4) {
                const float4 a = acc_lds4[(j * EPV + k) / 4][tid];
                ab = k % 4 == 0 ? a.x : k % 4 == 1 ? a.y : k % 4 == 2 ? a.z : a.w;
            } else if constexpr (LACC) {
                ab = acc_lds[j * EPV + k][tid];
            } else if constexpr (!RMS) {
                ab = acc_b[j][k];
            }
            if constexpr (G::ROWS > 1) {
                if (want_g) fold(ag);
                if constexpr (!RMS)
                    if (want_b) fold(ab);
            }
            vg[k] = ag;
            vb[k] = ab;
        }
        if (team == 0 && col_ok[j]) {
            if (want_g) put_row(part_g + prow * N + off, vg);
            if constexpr (!RMS)
                if (want_b) put_row(part_b + prow * N + off, vb);
        }
    }
}

// out[c] = sum over p = 0 .. P-1 of part[p * N + c], in a fixed order, for
// up to two (part, out) pairs: blockIdx.y = 0 takes (part_g, out_g), 1 takes
// (part_b, out_b); a null out skips its pair.  A workgroup of 64 * WAVES
// lanes takes 64 columns; wavefront w sums rows w, w + WAVES, w + 2 WAVES,
// ... into four accumulators in turn (row w + i WAVES goes to accumulator
// i mod 4), adds them as (a0 + a1) + (a2 + a3), then wavefront 0 adds the
// WAVES sums in order.  P = 0 gives zeros.
template <int WAVES>
__global__ __launch_bounds__(64 * WAVES)
void norm_colsum_kernel(const float* __restrict__ part_g, float* __restrict__ out_g,
                        const float* __restrict__ part_b, float* __restrict__ out_b, int64_t P, int N)
{
    __shared__ float q[WAVES][64];
    const float* part = blockIdx.y == 0 ? part_g : part_b;
    float* out = blockIdx.y == 0 ? out_g : out_b;
    if (out == nullptr) return;           // the same for the whole workgroup
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int64_t c = (int64_t)blockIdx.x * 64 + lane;
    float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
    if (c < N) {
        const float* col = part + c;
        int64_t p = w;
        for (; p + 3 * WAVES < P; p += 4 * WAVES) {
            a0 += col[p * N];
            a1 += col[(p + WAVES) * N];
            a2 += col[(p + 2 * WAVES) * N];
            a3 += col[(p + 3 * WAVES) * N];
        }
        if (p < P) a0 += col[p * N];
        if (p + WAVES < P) a1 += col[(p + WAVES) * N];
        if (p + 2 * WAVES < P) a2 += col[(p + 2 * WAVES) * N];
    }
    q[w][lane] = (a0 + a1) + (a2 + a3);
    __syncthreads();
    if (w == 0 && c < N) {
        float t = q[0][lane];
#pragma unroll
        for (int i = 1; i < WAVES; ++i) t += q[i][lane];
        out[c] = t;
    }
}
constexpr int kColsumWaves = 16;

// The same sums for few partial rows (P < 16): lane t of the grid takes
// columns 4t .. 4t + 3 (16-byte loads when N is a multiple of 4, else one
// column per lane) and adds rows 0, 1, ..., P - 1 in order.
template <bool V4>
__global__ __launch_bounds__(256)
void norm_colsum_narrow_kernel(const float* __restrict__ part_g, float* __restrict__ out_g,
                               const float* __restrict__ part_b, float* __restrict__ out_b, int64_t P, int N)
{
    const float* part = blockIdx.y == 0 ? part_g : part_b;
    float* out = blockIdx.y == 0 ? out_g : out_b;
    if (out == nullptr) return;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if constexpr (V4) {
        const int64_t c = t * 4;
        if (c >= N) return;
        float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        for (int64_t p = 0; p < P; ++p) {
            const float4 v = *reinterpret_cast<const float4*>(part + p * N + c);
            a.x += v.x;
            a.y += v.y;
            a.z += v.z;
            a.w += v.w;
        }
        out[c] = a.x;        // out is only 4-byte aligned
        out[c + 1] = a.y;
        out[c + 2] = a.z;
        out[c + 3] = a.w;
    } else {
        if (t >= N) return;
        float a = 0.0f;
        for (int64_t p = 0; p < P; ++p) a += part[p * N + t];
        out[t] = a;
    }
}

}  // namespace mi355norm
