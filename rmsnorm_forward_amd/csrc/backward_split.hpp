// backward_split.hpp -- LayerNorm / RMSNorm backward for rows too long for
// one workgroup ("CUDA 算子工程" ch. 7, section 7.7: the same formulas as
// backward.hpp, the row sums taken over chunks of the row).
//
// Per batch of rows (every row in one batch unless smaller batches are asked
// for), three kernels:
//
//   norm_bwd_split_sums_kernel    one workgroup per (row, chunk of 256 lanes x
//                                 2 vectors; 16 elements per lane on the
//                                 element-wise path): reads the chunk of dy and x
//                                 through the caches and stores the chunk's
//                                 (sum g, sum g xhat) -- (0, sum g x) for
//                                 RMSNorm -- to part[row * S + chunk].
//   norm_bwd_split_rowsum_kernel  one wavefront per row: the row's S chunk
//                                 sums added in a fixed order (lane l takes
//                                 chunks l, l + 64, ... into four
//                                 accumulators; then the wavefront
//                                 butterfly), one float2 per row.
//   norm_bwd_split_apply_kernel   a persistent grid of (column chunk of 256
//                                 lanes x VPL vectors, row group) workgroups:
//                                 each walks its rows (prefetching the next
//                                 row's dy, x, statistics and row sums), writes
//                                 dx and accumulates dgamma / dbeta for its
//                                 columns in registers, then adds them into
//                                 partial row `group` of part_g / part_b
//                                 (stored by the first batch, added to by the
//                                 later ones; every slot belongs to one
//                                 workgroup per batch).
//
// The column sums of the partial rows follow (norm_colsum_kernel), so
// dgamma and dbeta are summed in a fixed order throughout.
//
// norm_bwd_pass_kernel does it in one pass (dy and x read once, an ordinary
// launch), where the planner finds it faster or on request: teams of S
// workgroups, one per chunk of a row, walk
// the rows; each keeps its chunk of dy and x in registers, publishes its
// chunk sums in the row's slot for it (the forward single pass's protocol:
// a slot holds its value's bits inverted, zero meaning "not yet"), loads its
// next row's chunk, waits (bounded in time) until every slot of the row is
// filled, adds the row's S chunk sums in chunk order, forms dx from registers
// and accumulates dgamma / dbeta for its columns; partial row `team` holds
// them at the end.  If the wait runs out, the workgroup computes every
// chunk's sums of the row from dy and x itself (the same bits) and goes on,
// so nothing depends on the team being resident at once.
#pragma once

#include "prims.hpp"
#include "split.hpp"

namespace mi355norm {

// A lane's EPV consecutive columns of a partial row: written (or, with
// accumulate, added to) as 16-byte vectors when EPV and the row's alignment
// allow -- the partial rows may be dgamma / dbeta themselves, which need be
// 4-byte aligned only -- else one element at a time.
template <int EPV>
__device__ __forceinline__ void put_partial(float* dst, const float (&v)[EPV], bool vec, int accumulate) {
    if constexpr (EPV % 4 == 0) {
        if (vec) {
#pragma unroll
            for (int k = 0; k < EPV; k += 4) {
                float4 o = make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]);
                if (accumulate) {
                    const float4 a = *reinterpret_cast<const float4*>(dst + k);
                    o = make_float4(a.x + o.x, a.y + o.y, a.z + o.z, a.w + o.w);
                }
                *reinterpret_cast<float4*>(dst + k) = o;
            }
            return;
        }
    }
#pragma unroll
    for (int k = 0; k < EPV; ++k) dst[k] = accumulate ? dst[k] + v[k] : v[k];
}

template <class T, bool RMS, int WG, int VPL, int EPV>
__global__ __launch_bounds__(WG)
void norm_bwd_split_sums_kernel(const typename T::storage* __restrict__ dy,
                                const typename T::storage* __restrict__ x,
                                const typename T::storage* __restrict__ gamma,
                                const float* __restrict__ mean,
                                const float* __restrict__ rstd,
                                float2* __restrict__ part,
                                int64_t M, int N, int64_t ldy, int64_t ldx, int S)
{
    using V = Vec<T, EPV>;
    constexpr int CV = WG * VPL;   // vectors per chunk
    __shared__ float red[2][WG / 64];
    const int NV = N / EPV;
    const int64_t items = M * (int64_t)S;
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int64_t row = it / S;
        const int c = (int)(it - row * S);
        const typename T::storage* dyr = dy + row * ldy;
        const typename T::storage* xr = x + row * ldx;
        V dv[VPL], xv[VPL];
        bool ok[VPL];
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const unsigned v = (unsigned)(c * CV + j * WG) + threadIdx.x;
            ok[j] = (int)v < NV;
            if (ok[j]) {          // cached: the apply kernel reads them again soon
                dv[j].load(dyr + v * EPV);
                xv[j].load(xr + v * EPV);
            }
        }
        const float m = RMS ? 0.0f : mean[row];
        const float r = rstd[row];
        float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            if (!ok[j]) continue;
            const unsigned off = ((unsigned)(c * CV + j * WG) + threadIdx.x) * EPV;
            V gv;
            if (gamma != nullptr) gv.load(gamma + off);
#pragma unroll
            for (int k = 0; k < EPV; ++k) {
                const float g = dv[j].get(k) * (gamma != nullptr ? gv.get(k) : 1.0f);
                const float xh = RMS ? xv[j].get(k) : (xv[j].get(k) - m) * r;
                if constexpr (!RMS) s1 += g;
                s2 = __builtin_fmaf(g, xh, s2);
            }
        }
        // two exchanges on two slot sets: the second's barrier orders every
        // read of the first set before the next item writes it
        s1 = wg_sum<WG>(s1, red[0]);
        s2 = wg_sum<WG>(s2, red[1]);
        if (threadIdx.x == 0) part[row * S + c] = make_float2(s1, s2);
    }
}

// One row's chunk sums pr[0 .. S), summed by one wavefront into *out.
__device__ __forceinline__ void rowsum_one(const float2* __restrict__ pr, float2* __restrict__ out, int S)
{
    float2 a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = make_float2(0.0f, 0.0f);
    int c = lane_id();
    for (; c + 192 < S; c += 256) {
        float2 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = pr[c + 64 * i];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[i].x += v[i].x;
            a[i].y += v[i].y;
        }
    }
#pragma unroll
    for (int i = 0; i < 3; ++i)
        if (c + 64 * i < S) {
            const float2 v = pr[c + 64 * i];
            a[i].x += v.x;
            a[i].y += v.y;
        }
    float s1 = (a[0].x + a[1].x) + (a[2].x + a[3].x);
    float s2 = (a[0].y + a[1].y) + (a[2].y + a[3].y);
    s1 = team_sum<64>(s1);
    s2 = team_sum<64>(s2);
    if (lane_id() == 0) *out = make_float2(s1, s2);
}

// rows[r] = sum over c of part[r * S + c]; one wavefront per row, W rows
// per workgroup, rows grid-strided.  Lane l takes chunks l, l + 64,
// l + 128, ... into four accumulators in turn (chunk l + 64 i goes to
// accumulator i mod 4, so four loads are in flight), adds them as
// (a0 + a1) + (a2 + a3), then the wavefront butterfly: a fixed order.
template <int W>
__global__ __launch_bounds__(64 * W)
void norm_bwd_split_rowsum_kernel(const float2* __restrict__ part, float2* __restrict__ rows, int64_t M, int S)
{
    for (int64_t row = (int64_t)blockIdx.x * W + (threadIdx.x >> 6); row < M; row += (int64_t)gridDim.x * W)
        rowsum_one(part + row * S, rows + row, S);   // the row is the same for the whole wavefront
}

template <class T, bool RMS, int WG, int VPL, int EPV>
__global__ __launch_bounds__(WG)
void norm_bwd_split_apply_kernel(const typename T::storage* dy,      // dx may be written over dy or x
                                 const typename T::storage* x,
                                 const typename T::storage* __restrict__ gamma,
                                 const float* __restrict__ mean,
                                 const float* __restrict__ rstd,
                                 const float2* __restrict__ rows,    // [M] row sums
                                 typename T::storage* dx,
                                 float* __restrict__ part_g,         // [gridDim.x / A, N] or null
                                 float* __restrict__ part_b,         // [gridDim.x / A, N] or null
                                 int accumulate,                     // add into the partial rows
                                 int64_t M, int N, int64_t ldy, int64_t ldx, int64_t lddx, int A)
{
    using V = Vec<T, EPV>;
    using S = typename T::storage;
    constexpr int CV = WG * VPL;
    const int c = (int)(blockIdx.x % (unsigned)A);         // column chunk
    const int64_t grp = blockIdx.x / (unsigned)A;           // row group
    const int64_t groups = gridDim.x / (unsigned)A;
    const int NV = N / EPV;
    const float inv_n = 1.0f / (float)N;

    bool col_ok[VPL];
    V gam[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        const unsigned v = (unsigned)(c * CV + j * WG) + threadIdx.x;
        col_ok[j] = (int)v < NV;
        if (gamma != nullptr && col_ok[j]) {
            gam[j].load(gamma + v * EPV);
        } else {
            float one[EPV];
#pragma unroll
            for (int k = 0; k < EPV; ++k) one[k] = 1.0f;
            gam[j].set(one);
        }
    }
    float acc_g[VPL][EPV], acc_b[RMS ? 1 : VPL][EPV];
#pragma unroll
    for (int j = 0; j < VPL; ++j)
#pragma unroll
        for (int k = 0; k < EPV; ++k) {
            acc_g[j][k] = 0.0f;
            if constexpr (!RMS) acc_b[j][k] = 0.0f;
        }

    // a row's loads: its chunk of dy and x, its statistics and its row sums
    struct Row {
        V d[VPL], xx[VPL];
        float m, r;
        float2 s;
    };
    auto fetch = [&](int64_t row, Row& q) {
        if (row >= M) return;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const unsigned v = (unsigned)(c * CV + j * WG) + threadIdx.x;
            if (col_ok[j]) {          // nontemporal: the last read of dy and x
                q.d[j].load_stream(dy + row * ldy + v * EPV);
                q.xx[j].load_stream(x + row * ldx + v * EPV);
            }
        }
        q.m = RMS ? 0.0f : mean[row];
        q.r = rstd[row];
        q.s = rows[row];
    };
    // wait for a row's loads (see the row kernel: a wait placed after a
    // store would wait for the store too)
    auto ready = [&](Row& q) {
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            q.d[j].opaque();
            q.xx[j].opaque();
        }
        asm volatile("" : "+v"(q.m), "+v"(q.r), "+v"(q.s.x), "+v"(q.s.y));
    };
    auto work = [&](int64_t row, Row& q, Row& next) {
        const float c1 = q.s.x * inv_n;
        const float c2 = RMS ? q.r * q.r * q.r * (q.s.y * inv_n) : q.s.y * inv_n;
        V out[VPL];
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            if (!col_ok[j]) continue;
            float o[EPV];
#pragma unroll
            for (int k = 0; k < EPV; ++k) {
                const float dk = q.d[j].get(k);
                const float g = dk * gam[j].get(k);
                if constexpr (RMS) {
                    const float xk = q.xx[j].get(k);
                    o[k] = __builtin_fmaf(q.r, g, -xk * c2);
                    acc_g[j][k] = __builtin_fmaf(dk, xk * q.r, acc_g[j][k]);
                } else {
                    const float xh = (q.xx[j].get(k) - q.m) * q.r;
                    o[k] = q.r * ((g - c1) - xh * c2);
                    acc_g[j][k] = __builtin_fmaf(dk, xh, acc_g[j][k]);
                    acc_b[j][k] += dk;
                }
            }
            out[j].set(o);
        }
        ready(next);
        S* dxr = dx + row * lddx;
#pragma unroll
        for (int j = 0; j < VPL; ++j)
            if (col_ok[j]) out[j].put_stream(dxr + ((unsigned)(c * CV + j * WG) + threadIdx.x) * EPV);
    };
    Row qa, qb;
    fetch(grp, qa);
    ready(qa);
    for (int64_t row = grp; row < M;) {
        fetch(row + groups, qb);
        work(row, qa, qb);
        row += groups;
        if (row >= M) break;
        fetch(row + groups, qa);
        work(row, qb, qa);
        row += groups;
    }

    // this workgroup's columns of partial row `grp`
    const bool vg = (reinterpret_cast<uintptr_t>(part_g) & 15) == 0;
    const bool vb = (reinterpret_cast<uintptr_t>(part_b) & 15) == 0;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        if (!col_ok[j]) continue;
        const int64_t base = grp * (int64_t)N + ((int64_t)(c * CV + j * WG) + threadIdx.x) * EPV;
        if (part_g != nullptr) put_partial<EPV>(part_g + base, acc_g[j], vg, accumulate);
        if constexpr (!RMS)
            if (part_b != nullptr) put_partial<EPV>(part_b + base, acc_b[j], vb, accumulate);
    }
}

// Sum of a row's S chunk sums (read(c) gives chunk c's), in the fixed order
// of rowsum_one (lane l takes chunks l, l + 64, ... into four accumulators in
// turn, then the wavefront butterfly): the same bits in every wavefront.
template <class Read>
__device__ __forceinline__ float2 rowsum_read(Read&& read, int S) {
    float2 a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = make_float2(0.0f, 0.0f);
    int c = lane_id();
    for (; c + 192 < S; c += 256) {
        float2 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = read(c + 64 * i);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[i].x += v[i].x;
            a[i].y += v[i].y;
        }
    }
#pragma unroll
    for (int i = 0; i < 3; ++i)
        if (c + 64 * i < S) {
            const float2 v = read(c + 64 * i);
            a[i].x += v.x;
            a[i].y += v.y;
        }
    float s1 = (a[0].x + a[1].x) + (a[2].x + a[3].x);
    float s2 = (a[0].y + a[1].y) + (a[2].y + a[3].y);
    return make_float2(team_sum<64>(s1), team_sum<64>(s2));
}

template <class T, bool RMS, int WG, int VPL, int EPV>
__global__ __launch_bounds__(WG)
void norm_bwd_pass_kernel(const typename T::storage* dy,      // dx may be written over dy or x
                          const typename T::storage* x,
                          const typename T::storage* __restrict__ gamma,
                          const float* __restrict__ mean,
                          const float* __restrict__ rstd,
                          typename T::storage* dx,
                          float* __restrict__ part_g,         // [teams, N] or null
                          float* __restrict__ part_b,         // [teams, N] or null
                          unsigned long long* __restrict__ slots,   // [M, S] published chunk sums
                          unsigned* __restrict__ dep,         // row r's departures at dep[64 r]
                          int64_t M, int N, int64_t ldy, int64_t ldx, int64_t lddx, int S, int teams,
                          unsigned wait_ticks)
{
    using V = Vec<T, EPV>;
    using St = typename T::storage;
    constexpr int CV = WG * VPL;
    __shared__ float red[2][WG / 64];
    __shared__ float2 row_sums;               // of the row being finished
    __shared__ int late;
    const int tid = threadIdx.x;
    const int team = blockIdx.x / S;          // grid is exactly teams * S
    const int c = blockIdx.x - team * S;
    const int NV = N / EPV;
    const float inv_n = 1.0f / (float)N;

    // the columns of chunk cc: in-row flags and gamma (1 where absent)
    auto columns = [&](int cc, bool (&okv)[VPL], V (&gm)[VPL]) {
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const unsigned v = (unsigned)(cc * CV + j * WG) + tid;
            okv[j] = (int)v < NV;
            if (gamma != nullptr && okv[j]) {
                gm[j].load(gamma + v * EPV);
            } else {
                float one[EPV];
#pragma unroll
                for (int k = 0; k < EPV; ++k) one[k] = 1.0f;
                gm[j].set(one);
            }
        }
    };
    bool col_ok[VPL];
    V gam[VPL];
    columns(c, col_ok, gam);
    float acc_g[VPL][EPV], acc_b[RMS ? 1 : VPL][EPV];
#pragma unroll
    for (int j = 0; j < VPL; ++j)
#pragma unroll
        for (int k = 0; k < EPV; ++k) {
            acc_g[j][k] = 0.0f;
            if constexpr (!RMS) acc_b[j][k] = 0.0f;
        }

    struct Row {
        V d[VPL], xx[VPL];
        float m, r;
    };
    // chunk cc of dy and x of `row`, with its statistics
    auto fetch_chunk = [&](int64_t row, Row& q, int cc, const bool (&okv)[VPL]) {
        if (row >= M) return;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            unsigned v = (unsigned)(cc * CV + j * WG) + tid;
            // recomputed per row rather than kept: the compiler would hold
            // row-invariant addresses across the loop and spill
            asm volatile("" : "+v"(v));
            if (okv[j]) {          // nontemporal: dy and x are read once
                q.d[j].load_stream(dy + row * ldy + v * EPV);
                q.xx[j].load_stream(x + row * ldx + v * EPV);
            }
        }
        q.m = RMS ? 0.0f : mean[row];
        q.r = rstd[row];
    };
    auto fetch = [&](int64_t row, Row& q) { fetch_chunk(row, q, c, col_ok); };
    auto ready = [&](Row& q) {
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            q.d[j].opaque();
            q.xx[j].opaque();
        }
        asm volatile("" : "+v"(q.m), "+v"(q.r));
    };
    // (sum g, sum g xhat) -- (0, sum g x) for RMSNorm -- over a chunk, every
    // workgroup computing the same bits for the same chunk: contraction is
    // off, so each inlined copy performs exactly these IEEE operations (the
    // compiler would otherwise fuse some copies' products into dot-product
    // instructions that round differently)
    auto chunk_sums = [&](Row& q, const bool (&okv)[VPL], const V (&gm)[VPL]) {
#pragma clang fp contract(off)
        float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            if (!okv[j]) continue;
#pragma unroll
            for (int k = 0; k < EPV; ++k) {
                const float g = q.d[j].get(k) * gm[j].get(k);
                const float xh = RMS ? q.xx[j].get(k) : (q.xx[j].get(k) - q.m) * q.r;
                if constexpr (!RMS) s1 += g;
                s2 = __builtin_fmaf(g, xh, s2);
            }
        }
        // re-widen dy and x after the exchanges rather than keep fp32 copies
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            q.d[j].opaque();
            q.xx[j].opaque();
        }
        // two exchanges on two slot sets: the second's barrier orders every
        // read of the first set before the next write
        if constexpr (!RMS) s1 = wg_sum<WG>(s1, red[0]);
        s2 = wg_sum<WG>(s2, red[1]);
        return make_float2(s1, s2);
    };
    auto read = [](const unsigned long long* sl) { return [sl](int cc) { return slot_value(read_slot(sl + cc)); }; };
    // One row: chunk sums, publication, (the next row's loads), the wait,
    // the row sums, dx and the column accumulators.
    auto finish = [&](Row& q, int64_t row, auto&& during_wait, auto&& before_stores) {
        unsigned long long* rsl = slots + row * S;
        const float2 cs = chunk_sums(q, col_ok, gam);
        if (tid == 0) publish_slot(rsl + c, cs);
        during_wait();
        if (tid < 64) {
            const bool have = wait_slots(rsl, S, wait_ticks);
            if (have) {
                const float2 r = rowsum_read(read(rsl), S);
                if (tid == 0) row_sums = r;
                depart_row(dep + row * 64, rsl, S);
            }
            if (tid == 0) late = !have;
        }
        lds_barrier();
        if (late) {
            // recompute: every chunk's sums of the row from dy and x,
            // published (the bits its own workgroup publishes), then the sum
            for (int cc = 0; cc < S; ++cc) {
                bool okv[VPL];
                V gm[VPL];
                columns(cc, okv, gm);
                fetch_chunk(row, q, cc, okv);
                const float2 s = chunk_sums(q, okv, gm);
                if (tid == 0) publish_slot(rsl + cc, s);
                // RMSNorm's sums have one reduction, whose LDS slots the
                // next chunk's would otherwise rewrite while a wavefront
                // still reads them
                if constexpr (RMS) lds_barrier();
            }
            if (tid < 64) {
                const float2 r = rowsum_read(read(rsl), S);
                if (tid == 0) row_sums = r;
                depart_row(dep + row * 64, rsl, S);
            }
            lds_barrier();
            fetch(row, q);
            ready(q);
        }
        const float2 rs = row_sums;
        const float c1 = rs.x * inv_n;
        const float c2 = RMS ? q.r * q.r * q.r * (rs.y * inv_n) : rs.y * inv_n;
        V out[VPL];
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            if (!col_ok[j]) continue;
            float o[EPV];
#pragma unroll
            for (int k = 0; k < EPV; ++k) {
                const float dk = q.d[j].get(k);
                const float g = dk * gam[j].get(k);
                if constexpr (RMS) {
                    const float xk = q.xx[j].get(k);
                    o[k] = __builtin_fmaf(q.r, g, -xk * c2);
                    acc_g[j][k] = __builtin_fmaf(dk, xk * q.r, acc_g[j][k]);
                } else {
                    const float xh = (q.xx[j].get(k) - q.m) * q.r;
                    o[k] = q.r * ((g - c1) - xh * c2);
                    acc_g[j][k] = __builtin_fmaf(dk, xh, acc_g[j][k]);
                    acc_b[j][k] += dk;
                }
            }
            out[j].set(o);
        }
        before_stores();
        St* dxr = dx + row * lddx;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            unsigned o = ((unsigned)(c * CV + j * WG) + tid) * EPV;
            asm volatile("" : "+v"(o));
            if (col_ok[j]) out[j].put_stream(dxr + o);
        }
        lds_barrier();           // `row_sums` and `late` are rewritten for the next row
    };

    // two row register sets, the loop unrolled by two: the next row's loads
    // are issued during this row's wait and waited for before its stores
    Row qa, qb;
    fetch(team, qa);
    ready(qa);
    for (int64_t row = team; row < M;) {
        finish(qa, row, [&] { fetch(row + teams, qb); }, [&] { ready(qb); });
        row += teams;
        if (row >= M) break;
        finish(qb, row, [&] { fetch(row + teams, qa); }, [&] { ready(qa); });
        row += teams;
    }

    // this workgroup's columns of partial row `team`
    const bool vg = (reinterpret_cast<uintptr_t>(part_g) & 15) == 0;
    const bool vb = (reinterpret_cast<uintptr_t>(part_b) & 15) == 0;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        if (!col_ok[j]) continue;
        const int64_t base = (int64_t)team * N + ((int64_t)(c * CV + j * WG) + tid) * EPV;
        if (part_g != nullptr) put_partial<EPV>(part_g + base, acc_g[j], vg, 0);
        if constexpr (!RMS)
            if (part_b != nullptr) put_partial<EPV>(part_b + base, acc_b[j], vb, 0);
    }
}

}  // namespace mi355norm
