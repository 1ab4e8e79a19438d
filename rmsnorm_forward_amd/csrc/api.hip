// api.hip -- the C ABI (include/mi355norm.h): argument validation, choice of
// the row-to-workgroup mapping from (N, dtype, alignment), and launch.
//
// Mapping regimes, chosen by row length in 16-byte vectors (NV).  A lane
// holds four vectors for 2-byte types (32 elements) and two for fp32 (8
// elements); the team is as large as the row needs (at least 8 lanes), and
// for LayerNorm at most 2048 elements wide, beyond which lanes take up to 8
// vectors:
//   small rows  (bf16 N <= 1024, fp32 N <= 256): 8..32 lanes per row, 2..8
//               rows share a wavefront and reduce with DPP only;
//   mid rows    (up to 1024 lanes x 8 vectors: bf16 N <= 65536, fp32
//               N <= 32768): 64..1024 lanes per row, one LDS exchange per
//               reduction across the row's wavefronts;
//   long rows   (beyond 1024 lanes x 8 vectors): split across workgroups
//               in chunks; per-chunk partial statistics merged in chunk order
//               (Chan).  RMSNorm and fp32 LayerNorm on 16-byte vectors: a
//               single pass (ordinary launch, x read once; every chunk's
//               partial published in the row's slots, a bounded wait for the
//               row's other chunks, recomputing the row's partials from x
//               when the wait runs out; the next row's chunk loaded into LDS
//               during the wait).  LayerNorm with 16-bit I/O, the residual
//               add and element-wise rows: two kernels per batch of rows
//               holding about 256 MiB of x, partials (x read through the
//               caches), then merge + normalise (x read again, partly from
//               the Infinity Cache).
// x alone off a 16-byte boundary (a view into a wider buffer, any row
// stride), the other operands aligned and N filling whole vectors: the row
// tiles and the split rows' two kernels read x in aligned 16-byte blocks and
// realign them in registers (a DPP shift from the next lane, byte
// alignment), LayerNorm, RMSNorm and RMSNorm with FP8 output; the residual
// add takes the element-wise path.  Steady state, realigned vs aligned vs element-wise, us:
// LN bf16 16384 x 8192 105.2 / 88.8 / 228.7, RMS bf16 65536 x 2048 88.5 /
// 84.9 / 175.2, LN bf16 1024 x 32768 33.8 / 27.8 / 111.7, LN bf16 64 x 2^20
// (split) 80.5 / 64.6 / 264.2.
// Measured on MI355X in steady state (200 back-to-back launches): bf16
// 1024-wide RMSNorm 32x4 (2 rows per wavefront) 85.3 us vs 64x2 87.1, 16x8
// 95.1; bf16 2048-wide 64x4 87.6 vs 32x8 99.4; fp32 2048-wide 256x2 175.0
// vs 128x4 177.6, 64x8 189.6 (all before every load of a row was issued up
// front; with that, fp32 2048-wide RMSNorm 32x16 won, see make_plan).
//
// Test/benchmark hooks (environment, read per call):
//   MI355NORM_PATH = rows | split | split2 | split1 | splitpass
//                                       force the path (rows only if it fits;
//                                       split the split form make_plan picks;
//                                       split2 the two-kernel split; split1 or
//                                       splitpass the single pass, only if
//                                       every chunk of a row can be resident
//                                       at once, and not for the residual
//                                       add, which keeps two kernels; with x
//                                       alone misaligned it runs element-wise;
//                                       for the backward, split and split2
//                                       take the three-kernel split, split1 /
//                                       splitpass its single pass)
//   MI355NORM_SPLIT_BATCH = <bytes>     bytes of x per two-kernel split batch
//                                       (of dy and x in the split backward)
//   MI355NORM_TILE = <team>x<vpl>       force the row-kernel tile
//   MI355NORM_GRID = <n>                cap the number of workgroups
//   MI355NORM_WAIT_TICKS = <n>          bound of the single passes' waits
//                                       (100 MHz ticks)
//   MI355NORM_STAGGER = <n>             start delay of the second half of the
//                                       forward single pass's teams (ticks)
//   MI355NORM_FORCE_TIMEOUT = 1         make the single passes' waits run out
//                                       at once (every workgroup recomputes
//                                       its rows' partials from the inputs)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/mi355norm.h"
#include "dispatch.hpp"

using namespace mi355norm;

namespace {

__global__ void norm_zero_u32(unsigned* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

constexpr int64_t kMaxN = int64_t(1) << 24;
constexpr int64_t kMaxGrid = int64_t(1) << 20;

int elem_bytes(int dtype) { return dtype == NORM_F32 ? 4 : 2; }

// A matrix in memory: `rows` rows of `row` bytes, `ld` bytes apart (a
// vector is one row).
struct Mat {
    const void* p;
    int64_t rows, row, ld;
};

int64_t floor_div(int64_t a, int64_t b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }   // b > 0
int64_t ceil_div(int64_t a, int64_t b) { return -floor_div(-a, b); }

// Whether some byte belongs to both.  Exact when one of them is a single row
// or both have the same stride; otherwise any overlap of their spans counts.
bool overlaps(const Mat& a, const Mat& b) {
    if (!a.p || !b.p || a.rows <= 0 || b.rows <= 0 || a.row <= 0 || b.row <= 0) return false;
    const int64_t a0 = (int64_t)(uintptr_t)a.p, b0 = (int64_t)(uintptr_t)b.p;
    const int64_t a1 = a0 + (a.rows - 1) * a.ld + a.row, b1 = b0 + (b.rows - 1) * b.ld + b.row;
    if (a1 <= b0 || b1 <= a0) return false;
    if (a.rows == 1 && b.rows == 1) return true;
    if (b.rows == 1 || a.rows == 1) {
        // row i of the strided one meets the single row [s0, s0 + w)
        const Mat& m = b.rows == 1 ? a : b;
        const int64_t m0 = m.p == a.p ? a0 : b0;
        const int64_t s0 = b.rows == 1 ? b0 : a0, w = b.rows == 1 ? b.row : a.row;
        int64_t lo = floor_div(s0 - m0 - m.row, m.ld) + 1, hi = ceil_div(s0 + w - m0, m.ld) - 1;
        lo = std::max<int64_t>(lo, 0);
        hi = std::min<int64_t>(hi, m.rows - 1);
        return lo <= hi;
    }
    if (a.ld == b.ld) {
        // row i of a meets row j of b iff -b.row < (b0 - a0) + (j - i) * ld < a.row
        const int64_t d = b0 - a0, L = a.ld;
        int64_t lo = floor_div(-b.row - d, L) + 1, hi = ceil_div(a.row - d, L) - 1;
        lo = std::max<int64_t>(lo, -(a.rows - 1));
        hi = std::min<int64_t>(hi, b.rows - 1);
        return lo <= hi;
    }
    return true;
}

bool misaligned(const void* p, int a) { return p && ((uintptr_t)p % (uintptr_t)a) != 0; }

bool has_add(int op) { return op == OP_ADD_RMS || op == OP_ADD_RMS_Q8; }
bool has_q8(int op) { return op == OP_RMS_Q8 || op == OP_ADD_RMS_Q8; }

// Arguments of one call, row strides resolved (elements; bytes for FP8 y).
struct Args {
    int op, dtype;
    int64_t M, N;
    const void* x;
    const void* res;
    const void* gamma;
    const void* beta;
    void* y;
    void* hout;
    float* mean;
    float* rstd;
    float eps, scale;
    int64_t ldx, ldr, ldy, ldh;
};

int validate(const Args& a) {
    const int op = a.op;
    if (op < 0 || op >= kOps) return NORM_ERR_BAD_ARG;
    if (a.dtype != NORM_F32 && a.dtype != NORM_F16 && a.dtype != NORM_BF16) return NORM_ERR_BAD_DTYPE;
    const int64_t M = a.M, N = a.N;
    if (M < 0 || N < 1 || N > kMaxN) return NORM_ERR_BAD_SHAPE;
    const int e = elem_bytes(a.dtype);
    const int ye = has_q8(op) ? 1 : e;
    for (int64_t ld : {a.ldx, a.ldr, a.ldy, a.ldh})
        if (ld < N || ld > INT64_MAX / 8 || (M > 0 && M - 1 > (INT64_MAX / 8 - N) / ld)) return NORM_ERR_BAD_SHAPE;
    if (!(a.eps >= 0.0f) || std::isinf(a.eps)) return NORM_ERR_BAD_EPS;
    if (op != OP_LN && (a.beta || a.mean)) return NORM_ERR_BAD_ARG;
    if (has_q8(op) && !(a.scale > 0.0f && std::isfinite(a.scale) && std::isfinite(1.0f / a.scale)))
        return NORM_ERR_BAD_ARG;
    if (M == 0) return NORM_OK;
    if (!a.x || !a.y) return NORM_ERR_NULL_ARG;
    if (has_add(op) && (!a.res || !a.hout)) return NORM_ERR_NULL_ARG;
    if (misaligned(a.x, e) || misaligned(a.y, ye) || misaligned(a.gamma, e) || misaligned(a.beta, e) ||
        misaligned(a.res, e) || misaligned(a.hout, e) || misaligned(a.mean, 4) || misaligned(a.rstd, 4))
        return NORM_ERR_BAD_ARG;
    // in: 0 x, 1 res, 2 gamma, 3 beta;  out: 4 y, 5 hout, 6 mean, 7 rstd
    const Mat m[8] = {{a.x, M, N * e, a.ldx * e},   {a.res, M, N * e, a.ldr * e},
                      {a.gamma, 1, N * e, N * e},   {a.beta, 1, N * e, N * e},
                      {a.y, M, N * ye, a.ldy * ye}, {a.hout, M, N * e, a.ldh * e},
                      {a.mean, 1, M * 4, M * 4},    {a.rstd, 1, M * 4, M * 4}};
    const bool out[8] = {false, false, false, false, true, true, true, true};
    for (int i = 0; i < 8; ++i)
        for (int j = i + 1; j < 8; ++j) {
            if (!(out[i] || out[j]) || !overlaps(m[i], m[j])) continue;
            // with the residual add, y or the sum may be written exactly over
            // x or the residual (same pointer, stride and element size): each
            // element is read by the lane that writes it, before it writes
            const bool row_io = (i == 0 || i == 1) && (j == 4 || j == 5);
            if (has_add(op) && row_io && m[i].p == m[j].p && m[i].row == m[j].row && m[i].ld == m[j].ld)
                continue;
            return NORM_ERR_ALIAS;
        }
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
    int path = -1;        // -1 auto
    int split_mode = -1;  // -1 auto
    int team = 0, vpl = 0;
    int64_t grid = 0;
    unsigned wait_ticks = 100000;   // single passes: 1 ms
    unsigned stagger = 0;
    bool force_timeout = false;
    int64_t batch_bytes = 0;  // two-kernel split: bytes of x per batch (0: default)
};

Overrides read_overrides() {
    Overrides o;
    if (const char* s = std::getenv("MI355NORM_PATH")) {
        if (!std::strcmp(s, "rows")) o.path = PATH_ROWS;
        else if (!std::strcmp(s, "split")) o.path = PATH_SPLIT;
        else if (!std::strcmp(s, "split2")) { o.path = PATH_SPLIT; o.split_mode = SPLIT_TWO; }
        else if (!std::strcmp(s, "splitpass") || !std::strcmp(s, "split1")) {
            o.path = PATH_SPLIT;
            o.split_mode = SPLIT_PASS;
        }
    }
    if (const char* s = std::getenv("MI355NORM_FORCE_TIMEOUT")) o.force_timeout = std::atoi(s) != 0;
    if (const char* s = std::getenv("MI355NORM_WAIT_TICKS")) o.wait_ticks = (unsigned)std::strtoul(s, nullptr, 10);
    if (const char* s = std::getenv("MI355NORM_STAGGER")) o.stagger = (unsigned)std::strtoul(s, nullptr, 10);
    if (o.force_timeout) o.wait_ticks = 0;
    if (const char* s = std::getenv("MI355NORM_TILE")) {
        int t = 0, v = 0;
        if (std::sscanf(s, "%dx%d", &t, &v) == 2) { o.team = t; o.vpl = v; }
    }
    if (const char* s = std::getenv("MI355NORM_GRID")) o.grid = std::atoll(s);
    if (const char* s = std::getenv("MI355NORM_SPLIT_BATCH")) o.batch_bytes = std::atoll(s);
    return o;
}

bool tile_instantiated(int team, int vpl) {
    bool t = false, v = false;
    for (int c : kTeams) t |= c == team;
    for (int c : kVpls) v |= c == vpl;
    return t && v;
}

// one wavefront per row with 5 or 10 vectors per lane (forward row kernel only): for
// rows of 320 or 640 16-byte vectors when there are at most
// kWaveTileMaxRows rows
constexpr int kWaveTileVpls[] = {5, 10};
constexpr int64_t kWaveTileMaxRows = 4096;

// the forward row kernel also has the one-wavefront tiles
bool fwd_tile_instantiated(int team, int vpl) {
    if (team == 64)
        for (int c : kWaveTileVpls)
            if (c == vpl) return true;
    return tile_instantiated(team, vpl);
}

// How many workgroups of the forward's (bwd: the backward's) single-pass
// kernel the current device can hold at once (0 if no device is present, or
// if the forward's wide chunks are not built for the operation).  Cached per
// (device, dtype, op, vector width, direction, chunk width).
int64_t resident_capacity(int dtype, int op, int epv, bool bwd = false, bool wide = false) {
    static std::mutex mu;
    static int64_t cache[64][3][kOps][2][2][2];
    static bool known[64][3][kOps][2][2][2];
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) return 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    const int vi = epv == 1 ? 0 : 1;
    const int bi = bwd ? 1 : 0;
    const int wi = wide && !bwd ? 1 : 0;
    std::lock_guard<std::mutex> lock(mu);
    if (!known[dev][dtype][op][vi][bi][wi]) {
        int cus = 0;
        int64_t cap = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) {
            int per_cu;
            const int wg = wi ? kPassWideWG : kPassWG;
            if (bwd)
                per_cu = dtype == NORM_F32 ? bwd_pass_blocks_per_cu_f32(op, epv)
                         : dtype == NORM_BF16 ? bwd_pass_blocks_per_cu_bf16(op, epv)
                                              : bwd_pass_blocks_per_cu_f16(op, epv);
            else
                per_cu = dtype == NORM_F32 ? pass_blocks_per_cu_f32(op, epv, wg)
                         : dtype == NORM_BF16 ? pass_blocks_per_cu_bf16(op, epv, wg)
                                              : pass_blocks_per_cu_f16(op, epv, wg);
            cap = int64_t(per_cu) * cus;
        }
        cache[dev][dtype][op][vi][bi][wi] = cap;
        known[dev][dtype][op][vi][bi][wi] = true;
    }
    return cache[dev][dtype][op][vi][bi][wi];
}

// Returns NORM_OK and fills *p, or NORM_ERR_BAD_ARG if an override cannot run.
// realign: x is read through the realigned row kernel (aligned must be set)
int make_plan(int op, int64_t M, int64_t N, int dtype, bool aligned, const Overrides& o, Plan* p,
              bool realign = false) {
    const int e = elem_bytes(dtype);
    std::memset(p, 0, sizeof *p);
    p->epv = aligned ? 16 / e : 1;
    const int64_t NV = N / p->epv;
    // any instantiated tile can hold up to 1024 x 16 vectors, but 16 full
    // 16-byte vectors per lane spill (bf16 1024 x 131072: 205 us vs 125 us
    // split), so the automatic choice keeps 16-byte rows at 8 per lane
    const bool fits_rows = NV <= int64_t(kMaxTeam) * kMaxVpl;
    const bool rows_auto = NV <= int64_t(kMaxTeam) * (p->epv == 1 ? kMaxVpl : 8);
    int path = rows_auto ? PATH_ROWS : PATH_SPLIT;
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
            if (!fwd_tile_instantiated(team, vpl) || int64_t(team) * vpl < NV) return NORM_ERR_BAD_ARG;
        } else {
            int per_lane = e == 2 ? 4 : 2;
            // RMSNorm with 16-bit I/O past 512 vectors a row: two vectors per
            // lane (steady state, us, 4 vs 2 per lane, bf16: 16384 x 6144 66.8
            // vs 65.1, 16384 x 8192 90.7 vs 85.6, 65536 x 8192 361.4 vs 343.0,
            // 8192 x 16384 88.7 vs 87.7; fp16 16384 x 8192 89.3 vs 86.8; level
            // at 4096 wide; realigned x too: bf16 16384 x 8192 89.2 vs 87.7).
            // Not with the residual add (level or slower: bf16 8192 x 12288
            // 133.3 vs 137.0) or the FP8 output (below).
            if (op == OP_RMS && e == 2 && p->epv > 1 && NV > 512) per_lane = 2;
            // RMSNorm with FP8 output past 1024 vectors a row: eight vectors
            // per lane (teams of 256 lanes and under take the hoisted
            // schedule): bf16 8192 x 10240 46.1 us vs 53.9, 8192 x 12288 52.9
            // vs 61.5, 8192 x 16384 67.7 vs 78.2, 4096 x 32768 77.2 vs 83.5;
            // fp32 16384 x 8192 107.8 vs 116.7; at 1024 vectors 8 per lane
            // lost (bf16 16384 x 8192 66.4 vs 65.4).  Not measured with
            // realigned x, which keeps the four.
            if (op == OP_RMS_Q8 && p->epv > 1 && NV > 1024 && !realign) per_lane = 8;
            team = next_pow2((NV + per_lane - 1) / per_lane);
            if (team < 8) team = 8;
            if (team > kMaxTeam) team = kMaxTeam;
            // LayerNorm keeps a team's vector row at <= 2048 elements and
            // grows the vectors per lane instead (bf16 N = 16384: 256 x 8
            // 92.6 us vs 512 x 4 99.9; fp32 N = 8192: 512 x 4 46.9 vs
            // 1024 x 2 49.7), up to 8 per lane
            if (op == OP_LN && p->epv > 1) {
                const int cap = 2048 / p->epv;
                if (team > cap) team = cap;
                while ((NV + team - 1) / team > 8 && team < kMaxTeam) team *= 2;
            }
            vpl = round_vpl((NV + team - 1) / team);
            // few rows whose 16-byte vectors fill one wavefront x 5 or 10
            // exactly: one wavefront per row (no LDS exchange, every load
            // of the row issued at once) beats the ragged wider tile
            // (steady state, us, LN bf16 4096 x 5120: 64 x 10 14.7 vs
            // 256 x 4 18.4; 2048 x 5120 9.4 vs 11.0; LN bf16 4096 x 2560:
            // 64 x 5 9.0 vs 128 x 4 11.0; from 8192 rows on it is level or
            // slower: RMS bf16 8192 x 5120 32.5 vs 30.0)
            // (realigned x too: 4096 x 5120 64 x 10 21.5 us, 512 x 2 21.9,
            // 256 x 4 22.4)
            if (p->epv > 1 && M <= kWaveTileMaxRows)
                for (int c : kWaveTileVpls)
                    if (NV == int64_t(64) * c) { team = 64; vpl = c; }
            // RMSNorm fp32 rows of 2048: two rows per wavefront, 16 vectors
            // per lane (every load issued up front) beat one row per
            // wavefront in three separate runs (65536 x 2048, us: 170.3 vs
            // 172.2, 173.4 vs 174.8, 169.6 vs 171.4).  Not taken elsewhere:
            // bf16 rows of 2048 32 x 8 86.4 vs 64 x 4 84.5; fp32 rows of
            // 1024 16 x 16 172.8 vs 128 x 2 170.5, of 4096 64 x 16 171.5 vs
            // 512 x 2 170.4; the residual add would hold x and the residual
            // (128 VGPRs) before its first use
            // (not with realigned x: 32 x 16 209 us, 256 x 2 177.5)
            if (op == OP_RMS && dtype == NORM_F32 && p->epv == 4 && NV == 512 && !realign) {
                team = 32;
                vpl = 16;
            }
        }
        p->team = team;
        p->vpl = vpl;
        p->wg = team >= 256 ? team : 256;
        p->rows_per_wg = p->wg / team;
        p->work = (M + p->rows_per_wg - 1) / p->rows_per_wg;
    } else {
        // The single pass (x read once) is the automatic choice for RMSNorm
        // and fp32 LayerNorm rows of 16-byte vectors, where it beat the two
        // kernels (steady state, us, two kernels vs single pass: RMS bf16
        // 64 x 2^20 58.9 vs 53.9, 512 x 2^18 118.9 vs 102.2, 2048 x 2^18
        // 468.9 vs 392.0; RMS f32 256 x 2^20 469.7 vs 396.2; LN f32
        // 64 x 2^20 119.4 vs 113.5, 256 x 2^20 477.3 vs 429.8).  LayerNorm
        // with 16-bit I/O takes it only for few rows per team (see
        // kPassLn16MaxRowsPerTeam).  The residual add keeps two kernels.
        // The pass runs when every chunk of a row can be resident; asked for
        // and impossible, the call fails; chosen automatically and
        // impossible (no device, say), the two kernels run.  Realigned x
        // takes the two kernels: the pass kernel has no registers to spare
        // for the realignment (LayerNorm bf16: 121 VGPRs of 128).
        // Rows of at least kPassWideMinChunks wide chunks take them when a
        // row's worth can be resident (RMSNorm, fp32 LayerNorm).  LayerNorm
        // with 16-bit I/O takes the pass only when each team has at most
        // kPassLn16MaxRowsPerTeam rows to walk.
        const bool ln16 = op == OP_LN && dtype != NORM_F32;
        const bool pass_auto = o.split_mode < 0 && p->epv > 1 && !realign;
        const bool try_pass = (o.split_mode == SPLIT_PASS || pass_auto) && !has_add(op);
        const int64_t wv = int64_t(kPassWideWG) * kPassVPL;
        const int64_t wchunks = (NV + wv - 1) / wv;
        const bool wide_shape = p->epv > 1 && (op != OP_LN || dtype == NORM_F32) && NV >= kPassWideMinChunks * wv;
        const bool wide = try_pass && wide_shape && resident_capacity(dtype, op, p->epv, false, true) >= wchunks;
        const int pwg = wide ? kPassWideWG : kPassWG;
        const int64_t pv = int64_t(pwg) * kPassVPL;
        const int64_t pchunks = (NV + pv - 1) / pv;
        const int64_t cap = try_pass ? resident_capacity(dtype, op, p->epv, false, wide) : 0;
        if (o.split_mode == SPLIT_PASS && !has_add(op) && cap < pchunks) return NORM_ERR_BAD_ARG;
        const bool few_rows = cap >= pchunks && M <= int64_t(kPassLn16MaxRowsPerTeam) * (cap / pchunks);
        if (try_pass && cap >= pchunks && (o.split_mode == SPLIT_PASS || !ln16 || few_rows)) {
            p->split_mode = SPLIT_PASS;
            p->wg = pwg;
            p->vpl = kPassVPL;
            p->chunks = (int)pchunks;
            p->teams = (int)std::min<int64_t>(M, cap / pchunks);
            p->batch_rows = M;
            p->work = M * p->chunks;
        } else {
            const int64_t cv = int64_t(kStatsWG) * kStatsVPL;
            const int64_t av = int64_t(kApplyWG) * kApplyVPL;
            p->split_mode = SPLIT_TWO;
            p->wg = kStatsWG;
            p->vpl = kStatsVPL;
            p->chunks = (int)((NV + cv - 1) / cv);
            p->apply_chunks = (int)((NV + av - 1) / av);
            const int64_t bb = o.batch_bytes > 0 ? o.batch_bytes : kSplitBatchBytes;
            const int64_t rows = bb / (N * e);
            p->batch_rows = std::min<int64_t>(M, rows > 0 ? rows : 1);
            p->work = p->batch_rows * p->chunks;   // per launch
        }
    }
    int64_t cap = o.grid > 0 ? o.grid : kMaxGrid;
    p->grid = p->work < cap ? p->work : cap;
    if (p->path == PATH_SPLIT && p->split_mode == SPLIT_PASS) p->grid = int64_t(p->teams) * p->chunks;
    if (p->path == PATH_SPLIT && p->split_mode == SPLIT_TWO) {
        const int64_t aw = p->batch_rows * p->apply_chunks;
        p->apply_grid = aw < cap ? aw : cap;
    }
    return NORM_OK;
}

// Workspace of the split-row path, one per (device, stream), kept across
// calls.  Calls on one stream run in stream order, so they can share it;
// calls on different streams get different buffers.  Layout: barrier
// counters first, at a fixed base (their capacity fixed per allocation), then
// the per-chunk partials.  Everything is zero when allocated, and the
// single-pass kernel leaves every counter it used at zero when it finishes,
// so counters are zero at the start of every call whatever its shape.
// Growing (only on a new largest call) allocates a larger buffer and keeps the
// old one until the process exits: work already queued on the stream, and any
// HIP graph captured with it, go on using the old buffer, so nothing waits and
// no captured pointer dangles.
struct Workspace {
    unsigned* sync;   // single pass: >= 64 counters per row of a launch
    float2* part;     // >= rows * chunks partials
};

// The HIP failure behind the calling thread's most recent NORM_ERR_HIP.
thread_local char g_last_error[192] = "";

bool hip_ok(hipError_t e, const char* what) {
    if (e == hipSuccess) return true;
    std::snprintf(g_last_error, sizeof g_last_error, "%s: %s (%s, code %d)", what, hipGetErrorName(e),
                  hipGetErrorString(e), (int)e);
    return false;
}

bool stream_workspace(hipStream_t stream, size_t sync_words, size_t part_bytes, Workspace* out) {
    struct Buf { void* ptr; size_t sync_words; size_t part_bytes; };   // sync_words >= 64 * M
    static std::mutex mu;
    static std::map<std::pair<int, hipStream_t>, Buf> bufs;
    static std::vector<void*> retired;   // outgrown workspaces, never freed
    int dev = 0;
    if (!hip_ok(hipGetDevice(&dev), "hipGetDevice")) return false;
    std::lock_guard<std::mutex> lock(mu);
    Buf& b = bufs[{dev, stream}];
    if (!b.ptr || b.sync_words < sync_words || b.part_bytes < part_bytes) {
        if (b.ptr) retired.push_back(b.ptr);
        const size_t sw = std::max({sync_words, 2 * b.sync_words, size_t(4096)});
        const size_t pb = std::max({part_bytes, 2 * b.part_bytes, size_t(1) << 20});
        const size_t sync_bytes = (sw * sizeof(unsigned) + 255) & ~size_t(255);
        const size_t total = sync_bytes + ((pb + 255) & ~size_t(255));
        b = Buf{nullptr, 0, 0};
        void* ptr = nullptr;
        if (!hip_ok(hipMalloc(&ptr, total), "hipMalloc (workspace)")) return false;
        const size_t words = total / sizeof(unsigned);
        hipLaunchKernelGGL(norm_zero_u32, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                           static_cast<unsigned*>(ptr), (int64_t)words);
        if (!hip_ok(hipGetLastError(), "launch of the workspace fill kernel")) {
            (void)hipFree(ptr);
            return false;
        }
        b = Buf{ptr, sync_bytes / sizeof(unsigned), total - sync_bytes};
    }
    out->sync = static_cast<unsigned*>(b.ptr);
    out->part = reinterpret_cast<float2*>(static_cast<char*>(b.ptr) + b.sync_words * sizeof(unsigned));
    return true;
}

// Scratch of the allocation-free entry point (norm_fwd_noalloc): the
// partials of the two-kernel split, in a fixed array every GPU the library
// runs on holds until the process ends.  Calls of that entry point on one GPU
// share it, so calls that overlap on one GPU race.  In host code `scratch`
// names a host-side stand-in; kernels get the device address looked up below.
constexpr size_t kScratchBytes = size_t(1) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The device address of `scratch` on the current device, looked up once per
// device (that device current) and kept; nullptr (norm_last_error set) on
// failure.
void* scratch_address() {
    static std::mutex mu;
    static void* addr[64];
    int dev = 0;
    if (!hip_ok(hipGetDevice(&dev), "hipGetDevice")) return nullptr;
    if (dev < 0 || dev >= 64) {
        std::snprintf(g_last_error, sizeof g_last_error, "device %d: scratch is kept for devices 0..63", dev);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        if (!hip_ok(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress (scratch)")) return nullptr;
        addr[dev] = p;
    }
    return addr[dev];
}

// The 16-byte vector path: every matrix row and vector starts on a vector
// boundary of its own type, and N fills whole vectors.
bool vector_aligned(const Args& a) {
    const int e = elem_bytes(a.dtype);
    const int epv = 16 / e;
    auto al = [](const void* q, int b) { return ((uintptr_t)q % (uintptr_t)b) == 0; };
    if ((a.N * e) % 16) return false;
    for (const void* q : {a.x, a.res, (const void*)a.hout, a.gamma, a.beta})
        if (!al(q, 16)) return false;
    if ((a.ldx * e) % 16 || (a.ldr * e) % 16 || (a.ldh * e) % 16) return false;
    if (has_q8(a.op)) return al(a.y, epv) && a.ldy % epv == 0;       // EPV one-byte codes
    return al(a.y, 16) && (a.ldy * e) % 16 == 0;
}

// The row kernel's realigned form: x (any element-aligned address and row
// stride) is read in aligned 16-byte blocks realigned in registers, while
// gamma, beta and y keep the vector path's alignment.  LayerNorm, RMSNorm and
// RMSNorm with FP8 output; N fills whole vectors.
bool realign_ok(const Args& a) {
    if (a.op != OP_LN && a.op != OP_RMS && a.op != OP_RMS_Q8) return false;
    const int e = elem_bytes(a.dtype);
    const int epv = 16 / e;
    auto al = [](const void* q, int b) { return ((uintptr_t)q % (uintptr_t)b) == 0; };
    if ((a.N * e) % 16 || !al(a.x, e)) return false;
    if (!al(a.gamma, 16) || !al(a.beta, 16)) return false;
    if (has_q8(a.op)) return al(a.y, epv) && a.ldy % epv == 0;
    return al(a.y, 16) && (a.ldy * e) % 16 == 0;
}

// noalloc: the two-kernel split's partials go to `scratch` (no allocation
// anywhere on the call's path); a call that needs more than it holds, or the
// single pass, is refused before any launch.
int run(const Args& a, void* stream, bool noalloc = false) {
    int st = validate(a);
    if (st != NORM_OK || a.M == 0) return st;
    const int op = a.op, dtype = a.dtype;
    const int64_t M = a.M, N = a.N;
    const int e = elem_bytes(dtype);
    Plan p;
    Overrides ov = read_overrides();
    // the single pass needs the workspace's slots: without allocation the
    // automatic choice is the two kernels (asked for, the pass is refused)
    if (noalloc && ov.split_mode < 0) ov.split_mode = SPLIT_TWO;
    // x alone misaligned: the realigned row kernel, or the realigned two
    // kernels for split rows; the single pass, asked for, runs element-wise
    const bool aligned = vector_aligned(a);
    bool realign = !aligned && realign_ok(a);
    st = make_plan(op, M, N, dtype, aligned || realign, ov, &p, realign);
    if (st == NORM_OK && realign && p.path == PATH_SPLIT && p.split_mode != SPLIT_TWO) {
        realign = false;
        st = make_plan(op, M, N, dtype, false, ov, &p);
    }
    if (st != NORM_OK) return st;
    NormCall c{a.x, a.res, a.gamma, a.beta, a.y, a.hout, a.mean, a.rstd, M, (int)N, a.eps, (hipStream_t)stream,
               has_q8(op) ? 1.0f / a.scale : 1.0f, Strides{a.ldx, a.ldr, a.ldy, a.ldh}};
    const int ye = has_q8(op) ? 1 : e;    // bytes per element of y
    hipError_t err;
    if (p.path == PATH_ROWS) {
        switch (dtype) {
        case NORM_F32: err = realign ? launch_rows_realigned_f32(op, c, p) : launch_rows_f32(op, c, p); break;
        case NORM_BF16: err = realign ? launch_rows_realigned_bf16(op, c, p) : launch_rows_bf16(op, c, p); break;
        default: err = realign ? launch_rows_realigned_f16(op, c, p) : launch_rows_f16(op, c, p); break;
        }
        return hip_ok(err, "row kernel launch") ? NORM_OK : NORM_ERR_HIP;
    }
    // split path: partials (two kernels) or the single pass's departure
    // counters and slots live in the workspace this (device, stream) keeps
    const bool pass = p.split_mode == SPLIT_PASS;
    const int64_t rows = p.batch_rows;   // rows per launch (two-kernel form: per pair)
    const Overrides o = read_overrides();
    Workspace w;
    // single pass: rows x 64 counter words, then rows x chunks 8-byte slots
    const size_t sync_words = pass ? size_t(rows) * (kSyncStride + 2 * size_t(p.chunks)) : 0;
    const size_t part_bytes = pass ? 0 : size_t(rows) * size_t(p.chunks) * sizeof(float2);
    if (noalloc) {
        if (pass) return NORM_ERR_BAD_ARG;
        if (part_bytes > kScratchBytes) return NORM_ERR_SCRATCH;
        void* base = scratch_address();
        if (!base) return NORM_ERR_HIP;
        w = Workspace{nullptr, static_cast<float2*>(base)};
    } else if (!stream_workspace(c.stream, sync_words, part_bytes, &w)) {
        return NORM_ERR_HIP;
    }
    float2* part = w.part;
    if (pass) {
        unsigned* dep = w.sync;
        auto* slots = reinterpret_cast<unsigned long long*>(w.sync + size_t(rows) * kSyncStride);
        switch (dtype) {
        case NORM_F32: err = launch_split_pass_f32(op, c, p, slots, dep, o.wait_ticks, o.stagger); break;
        case NORM_BF16: err = launch_split_pass_bf16(op, c, p, slots, dep, o.wait_ticks, o.stagger); break;
        default: err = launch_split_pass_f16(op, c, p, slots, dep, o.wait_ticks, o.stagger); break;
        }
    } else {
        // Row batches in stream order; each batch reuses the partials.
        err = hipSuccess;
        for (int64_t r0 = 0; r0 < M && err == hipSuccess; r0 += rows) {
            const int64_t mb = std::min(rows, M - r0);
            NormCall cb = c;
            cb.x = static_cast<const char*>(c.x) + r0 * c.ld.x * e;
            cb.y = static_cast<char*>(c.y) + r0 * c.ld.y * ye;
            if (c.res) cb.res = static_cast<const char*>(c.res) + r0 * c.ld.r * e;
            if (c.hout) cb.hout = static_cast<char*>(c.hout) + r0 * c.ld.h * e;
            cb.mean = c.mean ? c.mean + r0 : nullptr;
            cb.rstd = c.rstd ? c.rstd + r0 : nullptr;
            cb.M = mb;
            Plan pb = p;
            pb.grid = std::min(p.grid, mb * p.chunks);
            pb.apply_grid = std::min(p.apply_grid, mb * p.apply_chunks);
            switch (dtype) {
            case NORM_F32:
                err = realign ? launch_split_realigned_f32(op, cb, pb, part) : launch_split_f32(op, cb, pb, part);
                break;
            case NORM_BF16:
                err = realign ? launch_split_realigned_bf16(op, cb, pb, part) : launch_split_bf16(op, cb, pb, part);
                break;
            default:
                err = realign ? launch_split_realigned_f16(op, cb, pb, part) : launch_split_f16(op, cb, pb, part);
                break;
            }
        }
    }
    return hip_ok(err, pass ? "single-pass split kernel launch" : "two-kernel split launch") ? NORM_OK
                                                                                               : NORM_ERR_HIP;
}

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------

// Arguments of one backward call, row strides resolved (elements).
struct BwdArgs {
    bool rms;
    int dtype;
    int64_t M, N;
    const void* dy;
    const void* x;
    const void* gamma;
    const float* mean;
    const float* rstd;
    void* dx;
    float* dgamma;
    float* dbeta;
    int64_t lddy, ldx, lddx;
};

// The 16-byte vector path: every row start on a 16-byte boundary and N
// filling whole vectors.
bool bwd_vector_aligned(const BwdArgs& a) {
    const int e = elem_bytes(a.dtype);
    if ((a.N * e) % 16) return false;
    for (const void* q : {a.dy, a.x, a.gamma, (const void*)a.dx})
        if ((uintptr_t)q % 16) return false;
    return (a.lddy * e) % 16 == 0 && (a.ldx * e) % 16 == 0 && (a.lddx * e) % 16 == 0;
}

bool bwd_tile_ok(int team, int vpl, int epv) {
    return team >= kBwdMinTeam && tile_instantiated(team, vpl) && vpl * epv <= kBwdMaxElems;
}

// The backward grid: one 1024-lane workgroup per CU, each writing one
// partial row of dgamma / dbeta.  Measured on MI355X, LN bf16 16384 x 8192
// (one 1024 x 1 team per workgroup): 145.5 us at 256 workgroups, 152.3 at
// 512, 162.7 at 768; a second resident workgroup per CU does not fit, and
// more partial rows cost traffic.
constexpr int kBwdWgPerCu = 1;

int device_cus() {
    static std::mutex mu;
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (!cache[dev]) {
        int cus = 0;
        cache[dev] = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                             cus > 0 ? cus : 256;
    }
    return cache[dev];
}

// A row kernel tile for the backward: one 16-byte vector per lane (eight
// elements unaligned) as long as a team of 1024 lanes covers the row, more
// beyond, at most kBwdMaxElems elements per lane; teams of 8..1024 lanes in
// workgroups of 1024.  Measured (LN bf16 16384 x 8192, one workgroup per
// CU): 1024 x 1 145.5 us, 512 x 2 151.5.  Rows longer than 1024 x
// kBwdMaxElems (16384 when unaligned), fp32 rows that would need
// kBwdMaxElems elements per lane (RMSNorm; LayerNorm past
// kBwdF32RowsMaxLnVectors vectors), or any row with MI355NORM_PATH=split,
// take the split backward: chunk sums over kBwdSplitWG x bwd_sums_vpl
// vectors (measured, 256 x 2 against 256 x 8 / 4, one batch: LN bf16 64 x
// 2^20 124.6 / 131.0 / 127.8 us, 2048 x 65536 232.4 / 237.7 / 232.3), dx over chunks of kBwdSplitWG x kBwdSplitApplyVPL vectors in a
// grid of (chunk, row group) with about two workgroups per CU, all rows in
// one batch (measured, LN bf16 2048 x 65536: 244 us in one batch, 263 / 310
// / 406 us in batches of 256 / 128 / 64 MiB of dy and x; the apply kernel's
// second read of dy and x is no faster from the Infinity Cache, and every
// batch costs its launches and tails).  cus = 0 asks the device.
int make_bwd_plan(int64_t M, int64_t N, int dtype, bool rms, bool aligned, const Overrides& o, int cus,
                  Plan* p) {
    const int e = elem_bytes(dtype);
    std::memset(p, 0, sizeof *p);
    p->epv = aligned ? 16 / e : 1;
    const int64_t NV = N / p->epv;
    int team, vpl;
    if (o.team) {
        team = o.team;
        vpl = o.vpl;
        if (!bwd_tile_ok(team, vpl, p->epv) || int64_t(team) * vpl < NV) return NORM_ERR_BAD_ARG;
    } else {
        const int per_lane = p->epv == 1 ? 8 : 1;
        team = next_pow2((NV + per_lane - 1) / per_lane);
        team = std::max(team, kBwdMinTeam);
        team = std::min(team, kMaxTeam);
        vpl = round_vpl((NV + team - 1) / team);
        const bool f32_32 = e == 4 && vpl > 0 && vpl * p->epv == kBwdMaxElems;
        const bool f32_wide = f32_32 && (rms || NV > kBwdF32RowsMaxLnVectors);
        const bool forced_pass = o.path == PATH_SPLIT && o.split_mode == SPLIT_PASS;
        // the single pass by itself (kBwdPassMinRowsPerTeam): rows of
        // 16-byte vectors the row kernel would not take, or fp32 rows of 32
        // elements per lane, with enough rows per team
        const bool pass_shape = o.path < 0 && p->epv > 1 && (rms || dtype != NORM_F16) &&
                                (vpl < 0 || !bwd_tile_ok(team, vpl, p->epv) || f32_32);
        if (forced_pass || pass_shape) {
            const int64_t ccv = int64_t(kBwdPassWG) * kBwdPassVPL;
            const int64_t cchunks = (NV + ccv - 1) / ccv;
            const int64_t cap = resident_capacity(dtype, rms ? OP_RMS : OP_LN, p->epv, true);
            const int64_t teams = std::max<int64_t>(1, std::min<int64_t>(M, cap / std::max<int64_t>(1, cchunks)));
            const bool take = forced_pass || (cap >= cchunks && M >= int64_t(kBwdPassMinRowsPerTeam) * teams);
            if (forced_pass && cap < cchunks) return NORM_ERR_BAD_ARG;
            if (take) {
                p->path = PATH_SPLIT;
                p->split_mode = SPLIT_PASS;
                p->wg = kBwdPassWG;
                p->vpl = kBwdPassVPL;
                p->chunks = (int)cchunks;
                p->teams = (int)teams;
                p->batch_rows = M;
                p->work = M * p->chunks;
                p->grid = int64_t(p->teams) * p->chunks;
                return NORM_OK;
            }
        }
        if (o.path == PATH_SPLIT || vpl < 0 || !bwd_tile_ok(team, vpl, p->epv) || f32_wide) {
            const int64_t ncu = cus > 0 ? cus : device_cus();
            const int64_t sv = int64_t(kBwdSplitWG) * bwd_sums_vpl(p->epv);
            const int64_t av = int64_t(kBwdSplitWG) * kBwdSplitApplyVPL;
            p->path = PATH_SPLIT;
            p->wg = kBwdSplitWG;
            p->vpl = kBwdSplitApplyVPL;
            p->chunks = (int)((NV + sv - 1) / sv);
            p->apply_chunks = (int)((NV + av - 1) / av);
            const int64_t rows = o.batch_bytes > 0 ? o.batch_bytes / (2 * N * e) : M;
            p->batch_rows = std::max<int64_t>(1, std::min<int64_t>(M, rows));
            const int64_t gc = (2 * ncu + p->apply_chunks - 1) / p->apply_chunks;
            p->teams = (int)std::max<int64_t>(1, std::min<int64_t>(gc, p->batch_rows));
            p->work = p->batch_rows * p->chunks;
            p->grid = std::min<int64_t>(p->work, o.grid > 0 ? o.grid : kMaxGrid);
            p->apply_grid = int64_t(p->apply_chunks) * p->teams;
            return NORM_OK;
        }
    }
    p->path = PATH_ROWS;
    p->team = team;
    p->vpl = vpl;
    p->wg = kBwdWG;
    p->rows_per_wg = p->wg / team;
    p->work = (M + p->rows_per_wg - 1) / p->rows_per_wg;
    const int64_t cap = o.grid > 0 ? o.grid : int64_t(kBwdWgPerCu) * (cus > 0 ? cus : device_cus());
    p->grid = std::min(p->work, cap);
    return NORM_OK;
}

int validate_bwd(const BwdArgs& a) {
    if (a.dtype != NORM_F32 && a.dtype != NORM_F16 && a.dtype != NORM_BF16) return NORM_ERR_BAD_DTYPE;
    const int64_t M = a.M, N = a.N;
    if (M < 0 || N < 1 || N > kMaxN) return NORM_ERR_BAD_SHAPE;
    for (int64_t ld : {a.lddy, a.ldx, a.lddx})
        if (ld < N || ld > INT64_MAX / 8 || (M > 0 && M - 1 > (INT64_MAX / 8 - N) / ld)) return NORM_ERR_BAD_SHAPE;
    if (a.rms && (a.dbeta || a.mean)) return NORM_ERR_BAD_ARG;
    if (M > 0 && (!a.dy || !a.x || !a.dx || !a.rstd || (!a.rms && !a.mean))) return NORM_ERR_NULL_ARG;
    const int e = elem_bytes(a.dtype);
    if (misaligned(a.dy, e) || misaligned(a.x, e) || misaligned(a.gamma, e) || misaligned(a.dx, e) ||
        misaligned(a.mean, 4) || misaligned(a.rstd, 4) || misaligned(a.dgamma, 4) || misaligned(a.dbeta, 4))
        return NORM_ERR_BAD_ARG;
    // in: 0 dy, 1 x, 2 gamma, 3 mean, 4 rstd;  out: 5 dx, 6 dgamma, 7 dbeta
    const Mat m[8] = {{a.dy, M, N * e, a.lddy * e},  {a.x, M, N * e, a.ldx * e},  {a.gamma, 1, N * e, N * e},
                      {a.mean, 1, M * 4, M * 4},      {a.rstd, 1, M * 4, M * 4}, {a.dx, M, N * e, a.lddx * e},
                      {a.dgamma, 1, N * 4, N * 4},    {a.dbeta, 1, N * 4, N * 4}};
    for (int i = 0; i < 8; ++i)
        for (int j = i + 1; j < 8; ++j) {
            if (j < 5 || !overlaps(m[i], m[j])) continue;
            // dx may be written exactly over dy or x (same pointer and
            // stride): a lane loads the elements it owns from both before it
            // stores any of them
            if (j == 5 && i <= 1 && m[i].p == m[j].p && m[i].ld == m[j].ld) continue;
            return NORM_ERR_ALIAS;
        }
    return NORM_OK;
}

// The split backward: batches of rows in stream order, then the column sums.
// Workspace: the batch's chunk sums, its row sums, then the partial rows of
// dgamma and dbeta (p.teams rows of N each), which every batch adds to.
int run_bwd_split(const BwdArgs& a, const Plan& p, hipStream_t s) {
    const int64_t M = a.M, N = a.N;
    const int e = elem_bytes(a.dtype);
    const size_t part_elems = size_t(p.batch_rows) * size_t(p.chunks);
    // one row group: its partial rows are dgamma / dbeta themselves
    const bool direct = p.teams == 1 && M > 0;
    const size_t cols = direct ? 0 : size_t(p.teams) * size_t(N);
    const int ncol = (a.dgamma ? 1 : 0) + (a.dbeta ? 1 : 0);
    // the partial rows start 256-byte aligned (the column sum may read them
    // as 16-byte vectors)
    const size_t col_off = ((part_elems + size_t(p.batch_rows)) * sizeof(float2) + 255) & ~size_t(255);
    const bool pass = p.split_mode == SPLIT_PASS;
    Workspace w;
    // single pass: M x 64 counter words, then M x chunks 8-byte slots, in the
    // counter region
    const size_t sync_words = pass ? size_t(M) * (kSyncStride + 2 * size_t(p.chunks)) : 0;
    if (!stream_workspace(s, sync_words, col_off + cols * ncol * sizeof(float), &w)) return NORM_ERR_HIP;
    float2* part = w.part;
    float2* rows = part + part_elems;
    float* colbase = reinterpret_cast<float*>(reinterpret_cast<char*>(part) + col_off);
    float* pg = direct ? a.dgamma : a.dgamma ? colbase : nullptr;
    float* pb = direct ? a.dbeta : a.dbeta ? colbase + (a.dgamma ? cols : 0) : nullptr;
    const int op = a.rms ? OP_RMS : OP_LN;
    hipError_t err = hipSuccess;
    if (pass && M > 0) {
        // every row in one launch; slots and counters are zero at the start
        // of every call (see the forward's single pass)
        const Overrides o = read_overrides();
        unsigned* dep = w.sync;
        auto* slots = reinterpret_cast<unsigned long long*>(w.sync + size_t(M) * kSyncStride);
        BwdCall c{a.dy, a.x, a.gamma, a.mean, a.rstd, a.dx, pg, pb, M, (int)N, a.lddy, a.ldx, a.lddx, s};
        switch (a.dtype) {
        case NORM_F32: err = launch_bwd_pass_f32(op, c, p, slots, dep, o.wait_ticks); break;
        case NORM_BF16: err = launch_bwd_pass_bf16(op, c, p, slots, dep, o.wait_ticks); break;
        default: err = launch_bwd_pass_f16(op, c, p, slots, dep, o.wait_ticks); break;
        }
    }
    int64_t b = 0;
    for (int64_t r0 = 0; !pass && r0 < M && err == hipSuccess; r0 += p.batch_rows, ++b) {
        const int64_t mb = std::min(p.batch_rows, M - r0);
        BwdCall c{static_cast<const char*>(a.dy) + r0 * a.lddy * e, static_cast<const char*>(a.x) + r0 * a.ldx * e,
                  a.gamma, a.mean ? a.mean + r0 : nullptr, a.rstd + r0, static_cast<char*>(a.dx) + r0 * a.lddx * e,
                  pg, pb, mb, (int)N, a.lddy, a.ldx, a.lddx, s};
        Plan pb_ = p;
        pb_.teams = (int)std::min<int64_t>(p.teams, mb);
        // a shorter last batch uses fewer row groups: the partial rows it
        // does not reach keep what the earlier batches put there
        switch (a.dtype) {
        case NORM_F32: err = launch_bwd_split_f32(op, c, pb_, part, rows, b > 0); break;
        case NORM_BF16: err = launch_bwd_split_bf16(op, c, pb_, part, rows, b > 0); break;
        default: err = launch_bwd_split_f16(op, c, pb_, part, rows, b > 0); break;
        }
    }
    if (!hip_ok(err, "split backward launch")) return NORM_ERR_HIP;
    if ((a.dgamma || a.dbeta) && !direct &&
        !hip_ok(launch_colsum(pg ? pg : pb, pg ? a.dgamma : a.dbeta, pg ? pb : nullptr, pg ? a.dbeta : nullptr,
                              M > 0 ? p.teams : 0, (int)N, s),   // zeros when M = 0
                "column-sum launch"))
        return NORM_ERR_HIP;
    return NORM_OK;
}

int run_bwd(const BwdArgs& a, void* stream) {
    int st = validate_bwd(a);
    if (st != NORM_OK) return st;
    const int64_t M = a.M, N = a.N;
    const bool sums = a.dgamma || a.dbeta;
    Plan p;
    st = make_bwd_plan(M, N, a.dtype, a.rms, bwd_vector_aligned(a), read_overrides(), 0, &p);
    if (st != NORM_OK) return st;
    const hipStream_t s = (hipStream_t)stream;
    if (p.path == PATH_SPLIT) return run_bwd_split(a, p, s);
    float* pg = nullptr;
    float* pb = nullptr;
    const int64_t P = p.grid;   // partial rows: one per workgroup
    if (sums && P > 0) {
        Workspace w;
        const size_t per = size_t(P) * size_t(N);
        if (!stream_workspace(s, 0, per * sizeof(float) * ((a.dgamma && a.dbeta) ? 2 : 1), &w))
            return NORM_ERR_HIP;
        float* base = reinterpret_cast<float*>(w.part);
        pg = a.dgamma ? base : nullptr;
        pb = a.dbeta ? (a.dgamma ? base + per : base) : nullptr;
    }
    hipError_t err = hipSuccess;
    if (M > 0) {
        BwdCall c{a.dy, a.x, a.gamma, a.mean, a.rstd, a.dx, pg, pb, M, (int)N, a.lddy, a.ldx, a.lddx, s};
        const int op = a.rms ? OP_RMS : OP_LN;
        switch (a.dtype) {
        case NORM_F32: err = launch_bwd_f32(op, c, p); break;
        case NORM_BF16: err = launch_bwd_bf16(op, c, p); break;
        default: err = launch_bwd_f16(op, c, p); break;
        }
        if (!hip_ok(err, "backward row kernel launch")) return NORM_ERR_HIP;
    }
    // column sums of the partial rows (zeros when M = 0), both in one launch
    if (sums) {
        const bool g = a.dgamma != nullptr;
        err = launch_colsum(g ? pg : pb, g ? a.dgamma : a.dbeta, g ? pb : nullptr, g ? a.dbeta : nullptr, P,
                            (int)N, s);
        if (!hip_ok(err, "column-sum launch")) return NORM_ERR_HIP;
    }
    return NORM_OK;
}

}  // namespace

extern "C" {

int norm_fwd(const norm_args* args, void* stream) {
    if (!args) return NORM_ERR_NULL_ARG;
    const norm_args& g = *args;
    auto ld = [&](int64_t v) { return v == 0 ? g.N : v; };
    Args a{g.op, g.dtype, g.M, g.N, g.x, g.residual, g.gamma, g.beta, g.y, g.residual_out, g.mean, g.rstd,
           g.eps, g.scale, ld(g.ld_x), ld(g.ld_residual), ld(g.ld_y), ld(g.ld_residual_out)};
    return run(a, stream);
}

int norm_fwd_noalloc(const norm_args* args, void* stream) {
    if (!args) return NORM_ERR_NULL_ARG;
    const norm_args& g = *args;
    auto ld = [&](int64_t v) { return v == 0 ? g.N : v; };
    Args a{g.op, g.dtype, g.M, g.N, g.x, g.residual, g.gamma, g.beta, g.y, g.residual_out, g.mean, g.rstd,
           g.eps, g.scale, ld(g.ld_x), ld(g.ld_residual), ld(g.ld_y), ld(g.ld_residual_out)};
    return run(a, stream, true);
}

int ln_fwd(const void* x, const void* gamma, const void* beta, void* y, float* mean, float* rstd,
           int64_t M, int64_t N, float eps, int dtype, void* stream) {
    return run(Args{OP_LN, dtype, M, N, x, nullptr, gamma, beta, y, nullptr, mean, rstd, eps, 1.0f, N, N, N, N},
               stream);
}

int rms_fwd(const void* x, const void* gamma, const void* beta, void* y, float* mean, float* rstd,
            int64_t M, int64_t N, float eps, int dtype, void* stream) {
    return run(Args{OP_RMS, dtype, M, N, x, nullptr, gamma, beta, y, nullptr, mean, rstd, eps, 1.0f, N, N, N, N},
               stream);
}

int add_rms_fwd(const void* x, const void* residual, const void* gamma, void* y, void* residual_out,
                float* rstd, int64_t M, int64_t N, float eps, int dtype, void* stream) {
    return run(Args{OP_ADD_RMS, dtype, M, N, x, residual, gamma, nullptr, y, residual_out, nullptr, rstd, eps,
                    1.0f, N, N, N, N},
               stream);
}

int rms_fp8_fwd(const void* x, const void* gamma, void* y, float* rstd, int64_t M, int64_t N, float eps,
                float scale, int dtype, void* stream) {
    return run(Args{OP_RMS_Q8, dtype, M, N, x, nullptr, gamma, nullptr, y, nullptr, nullptr, rstd, eps, scale,
                    N, N, N, N},
               stream);
}

int add_rms_fp8_fwd(const void* x, const void* residual, const void* gamma, void* y, void* residual_out,
                    float* rstd, int64_t M, int64_t N, float eps, float scale, int dtype, void* stream) {
    return run(Args{OP_ADD_RMS_Q8, dtype, M, N, x, residual, gamma, nullptr, y, residual_out, nullptr, rstd, eps,
                    scale, N, N, N, N},
               stream);
}

int ln_bwd(const void* dy, const void* x, const void* gamma, const float* mean, const float* rstd, void* dx,
           float* dgamma, float* dbeta, int64_t M, int64_t N, int dtype, void* stream) {
    return run_bwd(BwdArgs{false, dtype, M, N, dy, x, gamma, mean, rstd, dx, dgamma, dbeta, N, N, N}, stream);
}

int rms_bwd(const void* dy, const void* x, const void* gamma, const float* rstd, void* dx, float* dgamma,
            int64_t M, int64_t N, int dtype, void* stream) {
    return run_bwd(BwdArgs{true, dtype, M, N, dy, x, gamma, nullptr, rstd, dx, dgamma, nullptr, N, N, N}, stream);
}

int norm_bwd(const norm_bwd_args* args, void* stream) {
    if (!args) return NORM_ERR_NULL_ARG;
    const norm_bwd_args& g = *args;
    if (g.op != NORM_OP_LN && g.op != NORM_OP_RMS) return NORM_ERR_BAD_ARG;
    auto ld = [&](int64_t v) { return v == 0 ? g.N : v; };
    return run_bwd(BwdArgs{g.op == NORM_OP_RMS, g.dtype, g.M, g.N, g.dy, g.x, g.gamma, g.mean, g.rstd, g.dx,
                           g.dgamma, g.dbeta, ld(g.ld_dy), ld(g.ld_x), ld(g.ld_dx)},
                   stream);
}

int norm_bwd_describe(int rms, int64_t M, int64_t N, int dtype, int aligned, char* buf, int buflen) {
    if (dtype != NORM_F32 && dtype != NORM_F16 && dtype != NORM_BF16) return NORM_ERR_BAD_DTYPE;
    if (M < 0 || N < 1 || N > kMaxN) return NORM_ERR_BAD_SHAPE;
    const int e = elem_bytes(dtype);
    Plan p;
    int st = make_bwd_plan(M, N, dtype, rms != 0, aligned && (N * e) % 16 == 0, read_overrides(), 0, &p);
    if (st != NORM_OK) return st;
    if (buf && buflen > 0 && p.path == PATH_SPLIT)
        std::snprintf(buf, (size_t)buflen,
                      "path=bwd_split mode=%s op=%s wg=%d sums_vpl=%d apply_vpl=%d epv=%d chunks=%d "
                      "apply_chunks=%d batch_rows=%lld grid=%lld apply_grid=%lld partial_rows=%d",
                      p.split_mode == SPLIT_PASS ? "pass" : "three", rms ? "rms" : "ln", p.wg,
                      p.split_mode == SPLIT_PASS ? p.vpl : bwd_sums_vpl(p.epv), p.vpl, p.epv, p.chunks, p.apply_chunks,
                      (long long)p.batch_rows, (long long)p.grid, (long long)p.apply_grid, p.teams);
    else if (buf && buflen > 0)
        std::snprintf(buf, (size_t)buflen,
                      "path=bwd op=%s team=%d vpl=%d epv=%d wg=%d rows_per_wg=%d grid=%lld work=%lld "
                      "partial_rows=%lld",
                      rms ? "rms" : "ln", p.team, p.vpl, p.epv, p.wg, p.rows_per_wg, (long long)p.grid,
                      (long long)p.work, (long long)p.grid);
    return NORM_OK;
}

const char* norm_status_str(int status) {
    switch (status) {
    case NORM_OK: return "ok";
    case NORM_ERR_NULL_ARG: return "x or y is NULL";
    case NORM_ERR_BAD_SHAPE:
        return "bad shape: need M >= 0, 1 <= N <= 2^24 and M*N*elem within int64";
    case NORM_ERR_BAD_DTYPE: return "unknown dtype (0 = f32, 1 = f16, 2 = bf16)";
    case NORM_ERR_BAD_EPS: return "eps must be finite and >= 0";
    case NORM_ERR_BAD_ARG: return "bad argument: misaligned pointer, beta/mean given to an RMSNorm, a bad FP8 scale, or an unusable override";
    case NORM_ERR_ALIAS: return "buffers overlap (in-place use is not supported)";
    case NORM_ERR_HIP: return "HIP runtime call or kernel launch failed";
    case NORM_ERR_SCRATCH:
        return "the call needs more than the 1 MiB fixed scratch of norm_fwd_noalloc (use norm_fwd)";
    }
    return "unknown status";
}

const char* norm_last_error(void) { return g_last_error; }

int norm_describe(int op, int64_t M, int64_t N, int dtype, int aligned, char* buf, int buflen) {
    if (op < 0 || op >= kOps) return NORM_ERR_BAD_ARG;
    if (dtype != NORM_F32 && dtype != NORM_F16 && dtype != NORM_BF16) return NORM_ERR_BAD_DTYPE;
    if (M < 0 || N < 1 || N > kMaxN) return NORM_ERR_BAD_SHAPE;
    const int e = elem_bytes(dtype);
    Plan p;
    const bool vec = aligned && (N * e) % 16 == 0;
    // aligned == 2: x alone off 16 bytes (the realigned row kernel, where the
    // plan is a row tile and the operation has that form)
    bool realign = vec && aligned == 2 && (op == OP_LN || op == OP_RMS || op == OP_RMS_Q8);
    int st = make_plan(op, M, N, dtype, vec && (aligned != 2 || realign), read_overrides(), &p, realign);
    if (st == NORM_OK && realign && p.path == PATH_SPLIT && p.split_mode != SPLIT_TWO) {
        realign = false;
        st = make_plan(op, M, N, dtype, false, read_overrides(), &p);
    }
    if (st != NORM_OK) return st;
    if (!buf || buflen <= 0) return NORM_OK;
    if (p.path == PATH_ROWS)
        std::snprintf(buf, (size_t)buflen,
                      "path=rows team=%d vpl=%d epv=%d wg=%d rows_per_wg=%d grid=%lld work=%lld%s",
                      p.team, p.vpl, p.epv, p.wg, p.rows_per_wg, (long long)p.grid, (long long)p.work,
                      realign ? " x=realigned" : "");
    else
        std::snprintf(buf, (size_t)buflen,
                      "path=split mode=%s wg=%d vpl=%d epv=%d chunks=%d apply_wg=%d apply_vpl=%d "
                      "apply_chunks=%d teams=%d batch_rows=%lld grid=%lld apply_grid=%lld work=%lld "
                      "workspace=%lld%s",
                      p.split_mode == SPLIT_PASS ? "pass" : "two", p.wg, p.vpl, p.epv, p.chunks,
                      p.split_mode == SPLIT_TWO ? kApplyWG : 0, p.split_mode == SPLIT_TWO ? kApplyVPL : 0,
                      p.apply_chunks, p.teams, (long long)p.batch_rows, (long long)p.grid,
                      (long long)p.apply_grid, (long long)p.work,
                      (long long)(p.batch_rows * p.chunks * 8 +
                                  (p.split_mode == SPLIT_PASS ? p.batch_rows * kSyncStride * 4 : 0)),
                      realign ? " x=realigned" : "");
    return NORM_OK;
}

}  // extern "C"
