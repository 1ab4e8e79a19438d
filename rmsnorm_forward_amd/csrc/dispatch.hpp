// dispatch.hpp -- host-side interface between the C ABI (api.hip) and the
// per-dtype kernel instantiation units (inst_*.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.hpp"

namespace mi355norm {

// Operations: LayerNorm, RMSNorm, residual add followed by RMSNorm, and the
// two RMSNorm forms with FP8 (E4M3) output.
enum { OP_LN = 0, OP_RMS = 1, OP_ADD_RMS = 2, OP_RMS_Q8 = 3, OP_ADD_RMS_Q8 = 4 };
constexpr int kOps = 5;

struct NormCall {
    const void* x;
    const void* res;     // OP_ADD_RMS: the residual added to x (else null)
    const void* gamma;
    const void* beta;
    void* y;
    void* hout;          // OP_ADD_RMS: where x + res is stored (else null)
    float* mean;
    float* rstd;
    int64_t M;
    int N;
    float eps;
    hipStream_t stream;
    float qinv;          // FP8 output: 1 / scale
    Strides ld;          // row strides of x, res, y, hout
};

// A backward call: dy, x, dx [M, N] (row strides ld*), gamma [N] or null,
// the forward's fp32 mean (LayerNorm) and rstd [M]; column partials of
// dgamma / dbeta go to part_g / part_b ([P, N] fp32, either may be null).
struct BwdCall {
    const void* dy;
    const void* x;
    const void* gamma;
    const float* mean;
    const float* rstd;
    void* dx;
    float* part_g;
    float* part_b;
    int64_t M;
    int N;
    int64_t ldy, ldx, lddx;
    hipStream_t stream;
};

enum { PATH_ROWS = 0, PATH_SPLIT = 1 };
// split rows: two kernels per batch (three for the backward) or one pass
enum { SPLIT_TWO = 0, SPLIT_PASS = 2 };

struct Plan {
    int path;       // PATH_ROWS or PATH_SPLIT
    int team;       // rows: lanes per row
    int vpl;        // vectors per lane
    int epv;        // elements per vector (16 bytes worth, or 1)
    int wg;         // threads per workgroup
    int rows_per_wg;
    int64_t grid;   // workgroups launched (grid-stride loops cover the rest)
    int chunks;     // split: chunks per row (two-kernel form: of the statistics kernel)
    int apply_chunks;     // two-kernel form: chunks per row of the normalising kernel
    int64_t apply_grid;   // two-kernel form: workgroups of the normalising kernel
    int64_t work;   // rows: row groups; split: M * chunks
    int split_mode; // SPLIT_TWO or SPLIT_PASS
    int teams;      // single pass: rows processed concurrently (grid = teams * chunks)
    int64_t batch_rows;  // two-kernel split: rows per pair of launches
};

// Tiles instantiated for the row kernel.
constexpr int kTeams[] = {4, 8, 16, 32, 64, 128, 256, 512, 1024};
constexpr int kVpls[] = {1, 2, 4, 8, 16};
constexpr int kMaxTeam = 1024;
constexpr int kMaxVpl = 16;
// backward: at most this many elements per lane (dy, x and two column
// accumulators live in registers); teams of 8 lanes and up; longer rows take
// the split backward
constexpr int kBwdMaxElems = 32;
// fp32 rows that need 32 elements per lane run faster split (RMSNorm from
// there on, LayerNorm past this many vectors per row)
constexpr int kBwdF32RowsMaxLnVectors = 6144;
// split backward: chunk sums over 256 lanes x 2 vectors (x 16 elements when
// element-wise), dx and the column accumulators over 256 lanes x 2 vectors;
// all rows in one batch unless MI355NORM_SPLIT_BATCH asks for smaller ones
constexpr int kBwdSplitWG = 256;
constexpr int kBwdSplitSumsVPL = 2;
constexpr int kBwdSplitSumsVPLElem = 16;
constexpr int bwd_sums_vpl(int epv) { return epv == 1 ? kBwdSplitSumsVPLElem : kBwdSplitSumsVPL; }
constexpr int kBwdSplitApplyVPL = 2;
// split backward in one pass: chunks of 1024 lanes x 2 vectors, one
// workgroup per chunk
constexpr int kBwdPassWG = 1024;
constexpr int kBwdPassVPL = 2;
// The backward's single pass is taken by itself for rows of 16-byte vectors
// that leave the row kernel (split rows, and fp32 rows of 32 elements per
// lane) when every chunk of a row can be resident and each team walks at
// least this many rows; LayerNorm with fp16 I/O keeps the three kernels.
// Measured on MI355X (steady state, us, three kernels or row kernel / single
// pass): LN bf16 4096 x 40000 295.1 / 255.8, 2048 x 65536 213.8 / 200.8,
// 512 x 2^18 216.2 / 204.9, 768 x 2^18 322.8 / 291.4, 128 x 2^20 219.5 /
// 215.8, 256 x 2^20 439.5 / 393.3; RMS bf16 2048 x 65536 209.7 / 176.6,
// 128 x 2^20 211.5 / 189.9; RMS fp16 2048 x 65536 212.1 / 185.5; LN / RMS
// fp32 4096 x 32768 427.4 / 320.9, 428.4 / 300.2; 64 x 2^20 208.4 / 199.2,
// 204.8 / 183.2; LN fp32 2048 x 65536 430.3 / 338.4; row kernel LN fp32
// 8192 x 20000 486.8 / 412.5, 4096 x 24576 309.3 / 248.9.  With fewer rows
// per team the teams' skew is not amortised (LN bf16 64 x 2^20, 16 rows per
// team, 111.4 / 123.8; 96 x 2^20 162.8 / 169.2; 16 x 2^22 112.5 / 150.4),
// and LayerNorm with fp16 I/O gained nothing (2048 x 65536 219.5 / 221.5,
// 512 x 2^18 218.2 / 224.0, 256 x 2^20 439.9 / 428.8).
constexpr int kBwdPassMinRowsPerTeam = 32;
constexpr int kBwdMinTeam = 8;
// backward workgroups: always 1024 lanes (16 wavefronts fill a CU's wave
// slots at up to 128 VGPRs), 1024 / team rows at once
constexpr int kBwdWG = 1024;
// Split-row chunk geometry: the two kernels of the two-kernel form (each
// its own chunk size), and the single pass (fewer, larger chunks: fewer
// partials to wait for per row).
#ifndef MI355_STATS_WG
#define MI355_STATS_WG 256
#endif
#ifndef MI355_STATS_VPL
#define MI355_STATS_VPL 8
#endif
#ifndef MI355_APPLY_WG
#define MI355_APPLY_WG 256
#endif
#ifndef MI355_APPLY_VPL
#define MI355_APPLY_VPL 8
#endif
constexpr int kStatsWG = MI355_STATS_WG;
constexpr int kStatsVPL = MI355_STATS_VPL;
constexpr int kApplyWG = MI355_APPLY_WG;
constexpr int kApplyVPL = MI355_APPLY_VPL;
// the forward's single pass: chunks of kPassWG lanes x kPassVPL vectors, two
// workgroups per CU (measured on MI355X, LN bf16 64 x 2^20, us, without /
// with the next row's chunk loaded into LDS during the wait: 512 x 8
// 66.6-68.6 / 64.6-65.9; 1024 x 8 72-78 / 68.6-68.9 (one per CU); 512 x 16
// 70-74 / 68.2-68.4; 512 x 4 79 / 74; 1024 x 4 84-89 / 72.7-72.9)
#ifndef MI355_PASS_WG
#define MI355_PASS_WG 512
#endif
#ifndef MI355_PASS_VPL
#define MI355_PASS_VPL 8
#endif
constexpr int kPassWG = MI355_PASS_WG;
constexpr int kPassVPL = MI355_PASS_VPL;
// Wide chunks (kPassWideWG lanes x kPassVPL vectors, one workgroup per CU)
// for RMSNorm and fp32 LayerNorm rows of at least kPassWideMinChunks of them:
// half the workgroups per row to wait on.  Measured on MI355X (steady state,
// us, 512 / 1024 lanes): RMS bf16 64 x 2^20 53.9 / 50.7, 256 x 2^20 198.8 /
// 195.4; RMS fp32 64 x 2^20 107.0 / 99.3, 256 x 2^20 395.2 / 353.1; FP8 out
// of bf16 / fp32 64 x 2^20 52.5 / 51.3, 81.9 / 74.1; LN fp32 64 x 2^20
// 113.7 / 111.4, 256 x 2^20 431.3 / 416.8.  Shorter rows keep 512 lanes:
// with few chunks a row's last one is mostly empty or the teams are too few
// (RMS bf16 4096 x 81920 260.3 / 306.3, 2048 x 98304 157.6 / 163.3, 256 x
// 2^19 101.7 / 102.3; LN fp32 512 x 2^18 203.5 / 224.9).
#ifndef MI355_PASS_WIDE_WG
#define MI355_PASS_WIDE_WG 1024
#endif
constexpr int kPassWideWG = MI355_PASS_WIDE_WG;
constexpr int kPassWideMinChunks = 16;
// LayerNorm with 16-bit I/O takes the single pass by itself only when every
// team walks at most this many rows: there the two kernels' second launch
// and second read of x cost more than the teams' wait.  Measured on MI355X
// (steady state, us, two kernels / single pass, rows per team): bf16 256 x
// 131072 34.4 / 29.5 (2), 128 x 2^18 34.1 / 29.5 (2), 64 x 2^19 35.0 / 30.2
// (2), 16 x 2^21 35.0 / 32.1 (2), 8 x 2^22 38.1 / 34.4 (2), 48 x 2^20 48.9 /
// 45.9 (3), 16 x 2^20 18.6 / 17.2 (1); fp16 64 x 2^19 34.4 / 30.9, 256 x
// 131072 34.6 / 31.0 (2).  From four rows per team the two are level or the
// two kernels win: bf16 64 x 2^20 63.9 / 63.5 (4), 512 x 131072 63.8 / 63.6
// (4), 16 x 2^22 69.0 / 72.4 (4), 128 x 2^20 123.6 / 126.1 (8), 512 x 2^18
// 122.9 / 124.9 (8); fp16 128 x 2^19 64.8 / 65.8 (4).
constexpr int kPassLn16MaxRowsPerTeam = 3;
// Two-kernel split: rows per pair of launches are chosen so that one batch of
// x (about this many bytes) mostly stays in the 256 MB Infinity Cache between the
// statistics pass and the normalising pass.
#ifndef MI355_SPLIT_BATCH_BYTES
#define MI355_SPLIT_BATCH_BYTES (int64_t(256) << 20)
#endif
constexpr int64_t kSplitBatchBytes = MI355_SPLIT_BATCH_BYTES;
// single passes: the departure counters of consecutive rows are 64 words
// (256 bytes) apart
constexpr int kSyncStride = 64;

hipError_t launch_rows_f32(int op, const NormCall& c, const Plan& p);
hipError_t launch_rows_bf16(int op, const NormCall& c, const Plan& p);
hipError_t launch_rows_f16(int op, const NormCall& c, const Plan& p);
// row kernel with realigned loads of x (LayerNorm, RMSNorm, RMSNorm with FP8
// output; 16-byte vectors; x misaligned, every other operand aligned)
hipError_t launch_rows_realigned_f32(int op, const NormCall& c, const Plan& p);
hipError_t launch_rows_realigned_bf16(int op, const NormCall& c, const Plan& p);
hipError_t launch_rows_realigned_f16(int op, const NormCall& c, const Plan& p);
// the same for the two-kernel split
hipError_t launch_split_realigned_f32(int op, const NormCall& c, const Plan& p, float2* ws);
hipError_t launch_split_realigned_bf16(int op, const NormCall& c, const Plan& p, float2* ws);
hipError_t launch_split_realigned_f16(int op, const NormCall& c, const Plan& p, float2* ws);
// two-kernel split: ws holds M*chunks partials
hipError_t launch_split_f32(int op, const NormCall& c, const Plan& p, float2* ws);
hipError_t launch_split_bf16(int op, const NormCall& c, const Plan& p, float2* ws);
hipError_t launch_split_f16(int op, const NormCall& c, const Plan& p, float2* ws);
// single-pass split (LayerNorm, RMSNorm and its FP8 form): slots holds
// M*chunks published partials and dep one departure counter per row, 64
// words apart, all zero before the launch and zero again after it; a row's
// wait is bounded by wait_ticks of the 100 MHz clock (0: recompute at once),
// and the second half of the teams starts `stagger` ticks late
hipError_t launch_split_pass_f32(int op, const NormCall& c, const Plan& p, unsigned long long* slots,
                                 unsigned* dep, unsigned wait_ticks, unsigned stagger);
hipError_t launch_split_pass_bf16(int op, const NormCall& c, const Plan& p, unsigned long long* slots,
                                  unsigned* dep, unsigned wait_ticks, unsigned stagger);
hipError_t launch_split_pass_f16(int op, const NormCall& c, const Plan& p, unsigned long long* slots,
                                 unsigned* dep, unsigned wait_ticks, unsigned stagger);
// backward row kernel with the plan's tile (op OP_LN or OP_RMS), grid p.grid
hipError_t launch_bwd_f32(int op, const BwdCall& c, const Plan& p);
hipError_t launch_bwd_bf16(int op, const BwdCall& c, const Plan& p);
hipError_t launch_bwd_f16(int op, const BwdCall& c, const Plan& p);
// split backward for one batch of c.M rows: chunk sums into part
// ([M, p.chunks]), row sums into rows ([M]), then dx and the column partials
// (p.teams rows of N, added to the existing ones when accumulate is set)
hipError_t launch_bwd_split_f32(int op, const BwdCall& c, const Plan& p, float2* part, float2* rows, int accumulate);
hipError_t launch_bwd_split_bf16(int op, const BwdCall& c, const Plan& p, float2* part, float2* rows, int accumulate);
hipError_t launch_bwd_split_f16(int op, const BwdCall& c, const Plan& p, float2* part, float2* rows, int accumulate);
// split backward in one pass over all c.M rows: chunk sums published in
// slots ([M, p.chunks], zero before and after), departure counters in dep
// (64 words apart), partial rows p.teams x N; a row's wait is bounded by
// wait_ticks of the 100 MHz clock (0: recompute at once)
hipError_t launch_bwd_pass_f32(int op, const BwdCall& c, const Plan& p, unsigned long long* slots, unsigned* dep,
                               unsigned wait_ticks);
hipError_t launch_bwd_pass_bf16(int op, const BwdCall& c, const Plan& p, unsigned long long* slots, unsigned* dep,
                                unsigned wait_ticks);
hipError_t launch_bwd_pass_f16(int op, const BwdCall& c, const Plan& p, unsigned long long* slots, unsigned* dep,
                               unsigned wait_ticks);
// workgroups of the single-pass split backward that fit on one CU at once
int bwd_pass_blocks_per_cu_f32(int op, int epv);
int bwd_pass_blocks_per_cu_bf16(int op, int epv);
int bwd_pass_blocks_per_cu_f16(int op, int epv);
// out_*[c] = sum of the P partial rows part_* of column c (fixed order), for
// dgamma and (out_b not null) dbeta in one launch
hipError_t launch_colsum(const float* part_g, float* out_g, const float* part_b, float* out_b, int64_t P, int N,
                         hipStream_t stream);
// workgroups of the forward's single-pass kernel that fit on one CU at once
int pass_blocks_per_cu_f32(int op, int epv, int wg);
int pass_blocks_per_cu_bf16(int op, int epv, int wg);
int pass_blocks_per_cu_f16(int op, int epv, int wg);

}  // namespace mi355norm
