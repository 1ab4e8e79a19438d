// api.hip -- the C ABI (include/mi355norm.h): argument validation, choice of
// the row-to-workgroup mapping from (N, dtype, alignment), and launch.
//
// Mapping regimes, chosen by row length in 16-byte vectors (NV).  Every lane
// holds four vectors for 2-byte types (32 elements) and two for fp32 (8
// elements); the team is as large as the row needs (at least 8 lanes):
//   small rows  (bf16 N <= 1024, fp32 N <= 256): 8..32 lanes per row, 2..8
//               rows share a wavefront and reduce with DPP only;
//   mid rows    (up to 1024 lanes): 64..1024 lanes per row, one LDS exchange
//               per reduction across the row's wavefronts; longer rows give
//               the 1024-lane team up to 16 vectors per lane;
//   long rows   (beyond 1024 lanes x 16 vectors): split across workgroups,
//               per-chunk partial statistics merged in chunk order (Chan) in
//               a second kernel.
// Measured on MI355X in steady state (200 back-to-back launches): bf16
// 1024-wide RMSNorm 32x4 (2 rows per wavefront) 85.3 us vs 64x2 87.1, 16x8
// 95.1; bf16 2048-wide 64x4 87.6 vs 32x8 99.4; fp32 2048-wide 256x2 175.0
// vs 128x4 177.6, 64x8 189.6.  More than four vectors per lane, or 4-lane
// teams, always lost.
//
// Test/benchmark hooks (environment, read per call):
//   MI355NORM_PATH = rows | split      force the path (rows only if it fits)
//   MI355NORM_TILE = <team>x<vpl>       force the row-kernel tile
//   MI355NORM_GRID = <n>                cap the number of workgroups
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/mi355norm.h"
#include "dispatch.hpp"

using namespace mi355norm;

namespace {

enum { OP_LN = 0, OP_RMS = 1 };

constexpr int64_t kMaxN = int64_t(1) << 24;
constexpr int64_t kMaxGrid = int64_t(1) << 20;

int elem_bytes(int dtype) { return dtype == NORM_F32 ? 4 : 2; }

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
    if (!a || !b || na <= 0 || nb <= 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

bool misaligned(const void* p, int a) { return p && ((uintptr_t)p % (uintptr_t)a) != 0; }

int validate(int op, const void* x, const void* gamma, const void* beta, const void* y,
             const float* mean, const float* rstd, int64_t M, int64_t N, float eps, int dtype) {
    if (dtype != NORM_F32 && dtype != NORM_F16 && dtype != NORM_BF16) return NORM_ERR_BAD_DTYPE;
    if (M < 0 || N < 1 || N > kMaxN) return NORM_ERR_BAD_SHAPE;
    const int e = elem_bytes(dtype);
    if (M > INT64_MAX / N / e) return NORM_ERR_BAD_SHAPE;
    if (!(eps >= 0.0f) || std::isinf(eps)) return NORM_ERR_BAD_EPS;
    if (op == OP_RMS && (beta || mean)) return NORM_ERR_BAD_ARG;
    if (M == 0) return NORM_OK;
    if (!x || !y) return NORM_ERR_NULL_ARG;
    if (misaligned(x, e) || misaligned(y, e) || misaligned(gamma, e) || misaligned(beta, e) ||
        misaligned(mean, 4) || misaligned(rstd, 4))
        return NORM_ERR_BAD_ARG;
    const int64_t nx = M * N * e, nv = N * e, ns = M * 4;
    struct R { const void* p; int64_t n; bool out; } r[6] = {
        {x, nx, false}, {gamma, nv, false}, {beta, nv, false},
        {y, nx, true}, {mean, ns, true}, {rstd, ns, true}};
    for (int i = 0; i < 6; ++i)
        for (int j = i + 1; j < 6; ++j)
            if ((r[i].out || r[j].out) && overlaps(r[i].p, r[i].n, r[j].p, r[j].n)) return NORM_ERR_ALIAS;
    return NORM_OK;
}

int next_pow2(int64_t v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

int round_vpl(int64_t v) {
    for (int c : kVpls)
        if (c >= v) return c;
    return -1;
}

// Environment hooks for tests and the benchmark.
struct Overrides {
    int path = -1;   // -1 auto
    int team = 0, vpl = 0;
    int64_t grid = 0;
};

Overrides read_overrides() {
    Overrides o;
    if (const char* s = std::getenv("MI355NORM_PATH")) {
        if (!std::strcmp(s, "rows")) o.path = PATH_ROWS;
        else if (!std::strcmp(s, "split")) o.path = PATH_SPLIT;
    }
    if (const char* s = std::getenv("MI355NORM_TILE")) {
        int t = 0, v = 0;
        if (std::sscanf(s, "%dx%d", &t, &v) == 2) { o.team = t; o.vpl = v; }
    }
    if (const char* s = std::getenv("MI355NORM_GRID")) o.grid = std::atoll(s);
    return o;
}

bool tile_instantiated(int team, int vpl) {
    bool t = false, v = false;
    for (int c : kTeams) t |= c == team;
    for (int c : kVpls) v |= c == vpl;
    return t && v;
}

// Returns NORM_OK and fills *p, or NORM_ERR_BAD_ARG if an override cannot run.
int make_plan(int op, int64_t M, int64_t N, int dtype, bool aligned, const Overrides& o, Plan* p) {
    (void)op;
    const int e = elem_bytes(dtype);
    std::memset(p, 0, sizeof *p);
    p->epv = aligned ? 16 / e : 1;
    const int64_t NV = N / p->epv;
    const bool fits_rows = NV <= int64_t(kMaxTeam) * kMaxVpl;
    int path = fits_rows ? PATH_ROWS : PATH_SPLIT;
    if (o.path == PATH_SPLIT) path = PATH_SPLIT;
    if (o.path == PATH_ROWS) {
        if (!fits_rows) return NORM_ERR_BAD_ARG;
        path = PATH_ROWS;
    }
    p->path = path;
    if (path == PATH_ROWS) {
        int team, vpl;
        if (o.team) {
            team = o.team;
            vpl = o.vpl;
            if (!tile_instantiated(team, vpl) || int64_t(team) * vpl < NV) return NORM_ERR_BAD_ARG;
        } else {
            const int per_lane = e == 2 ? 4 : 2;
            team = next_pow2((NV + per_lane - 1) / per_lane);
            if (team < 8) team = 8;
            if (team > kMaxTeam) team = kMaxTeam;
            vpl = round_vpl((NV + team - 1) / team);
        }
        p->team = team;
        p->vpl = vpl;
        p->wg = team >= 256 ? team : 256;
        p->rows_per_wg = p->wg / team;
        p->work = (M + p->rows_per_wg - 1) / p->rows_per_wg;
    } else {
        p->wg = kSplitWG;
        p->vpl = kSplitVPL;
        const int64_t cv = int64_t(kSplitWG) * kSplitVPL;
        p->chunks = (int)((NV + cv - 1) / cv);
        p->work = M * p->chunks;
    }
    int64_t cap = o.grid > 0 ? o.grid : kMaxGrid;
    p->grid = p->work < cap ? p->work : cap;
    return NORM_OK;
}

bool all_aligned16(const void* x, const void* g, const void* b, const void* y, int64_t N, int e) {
    auto a = [](const void* q) { return ((uintptr_t)q & 15) == 0; };
    return (N * e) % 16 == 0 && a(x) && a(y) && a(g) && a(b);
}

int run(int op, const void* x, const void* gamma, const void* beta, void* y, float* mean,
        float* rstd, int64_t M, int64_t N, float eps, int dtype, void* stream) {
    int st = validate(op, x, gamma, beta, y, mean, rstd, M, N, eps, dtype);
    if (st != NORM_OK || M == 0) return st;
    const int e = elem_bytes(dtype);
    Plan p;
    st = make_plan(op, M, N, dtype, all_aligned16(x, gamma, beta, y, N, e), read_overrides(), &p);
    if (st != NORM_OK) return st;
    NormCall c{x, gamma, beta, y, mean, rstd, M, (int)N, eps, (hipStream_t)stream};
    const bool rms = op == OP_RMS;
    hipError_t err;
    if (p.path == PATH_ROWS) {
        switch (dtype) {
        case NORM_F32: err = launch_rows_f32(rms, c, p); break;
        case NORM_BF16: err = launch_rows_bf16(rms, c, p); break;
        default: err = launch_rows_f16(rms, c, p); break;
        }
        return err == hipSuccess ? NORM_OK : NORM_ERR_HIP;
    }
    // split path: stream-ordered workspace of M * chunks partials
    float2* ws = nullptr;
    const size_t ws_bytes = size_t(M) * size_t(p.chunks) * sizeof(float2);
    if (hipMallocAsync(reinterpret_cast<void**>(&ws), ws_bytes, c.stream) != hipSuccess) return NORM_ERR_HIP;
    switch (dtype) {
    case NORM_F32: err = launch_split_f32(rms, c, p, ws); break;
    case NORM_BF16: err = launch_split_bf16(rms, c, p, ws); break;
    default: err = launch_split_f16(rms, c, p, ws); break;
    }
    const hipError_t ferr = hipFreeAsync(ws, c.stream);
    return (err == hipSuccess && ferr == hipSuccess) ? NORM_OK : NORM_ERR_HIP;
}

}  // namespace

extern "C" {

int ln_fwd(const void* x, const void* gamma, const void* beta, void* y, float* mean, float* rstd,
           int64_t M, int64_t N, float eps, int dtype, void* stream) {
    return run(OP_LN, x, gamma, beta, y, mean, rstd, M, N, eps, dtype, stream);
}

int rms_fwd(const void* x, const void* gamma, const void* beta, void* y, float* mean, float* rstd,
            int64_t M, int64_t N, float eps, int dtype, void* stream) {
    return run(OP_RMS, x, gamma, beta, y, mean, rstd, M, N, eps, dtype, stream);
}

const char* norm_status_str(int status) {
    switch (status) {
    case NORM_OK: return "ok";
    case NORM_ERR_NULL_ARG: return "x or y is NULL";
    case NORM_ERR_BAD_SHAPE: return "bad shape: need M >= 0, 1 <= N <= 2^24 and M*N*elem within int64";
    case NORM_ERR_BAD_DTYPE: return "unknown dtype (0 = f32, 1 = f16, 2 = bf16)";
    case NORM_ERR_BAD_EPS: return "eps must be finite and >= 0";
    case NORM_ERR_BAD_ARG: return "bad argument: misaligned pointer, beta/mean given to rms_fwd, or an unusable override";
    case NORM_ERR_ALIAS: return "buffers overlap (in-place use is not supported)";
    case NORM_ERR_HIP: return "HIP runtime call or kernel launch failed";
    }
    return "unknown status";
}

int norm_describe(int op, int64_t M, int64_t N, int dtype, int aligned, char* buf, int buflen) {
    if (op != OP_LN && op != OP_RMS) return NORM_ERR_BAD_ARG;
    if (dtype != NORM_F32 && dtype != NORM_F16 && dtype != NORM_BF16) return NORM_ERR_BAD_DTYPE;
    if (M < 0 || N < 1 || N > kMaxN) return NORM_ERR_BAD_SHAPE;
    const int e = elem_bytes(dtype);
    Plan p;
    int st = make_plan(op, M, N, dtype, aligned && (N * e) % 16 == 0, read_overrides(), &p);
    if (st != NORM_OK) return st;
    if (!buf || buflen <= 0) return NORM_OK;
    if (p.path == PATH_ROWS)
        std::snprintf(buf, (size_t)buflen,
                      "path=rows team=%d vpl=%d epv=%d wg=%d rows_per_wg=%d grid=%lld work=%lld",
                      p.team, p.vpl, p.epv, p.wg, p.rows_per_wg, (long long)p.grid, (long long)p.work);
    else
        std::snprintf(buf, (size_t)buflen,
                      "path=split wg=%d vpl=%d epv=%d chunks=%d grid=%lld work=%lld workspace=%lld",
                      p.wg, p.vpl, p.epv, p.chunks, (long long)p.grid, (long long)p.work,
                      (long long)(M * p.chunks * 8));
    return NORM_OK;
}

}  // extern "C"
