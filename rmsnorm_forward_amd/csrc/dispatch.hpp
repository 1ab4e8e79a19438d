// dispatch.hpp -- host-side interface between the C ABI (api.hip) and the
// per-dtype kernel instantiation units (inst_*.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355norm {

struct NormCall {
    const void* x;
    const void* gamma;
    const void* beta;
    void* y;
    float* mean;
    float* rstd;
    int64_t M;
    int N;
    float eps;
    hipStream_t stream;
};

enum { PATH_ROWS = 0, PATH_SPLIT = 1 };

struct Plan {
    int path;       // PATH_ROWS or PATH_SPLIT
    int team;       // rows: lanes per row
    int vpl;        // vectors per lane
    int epv;        // elements per vector (16 bytes worth, or 1)
    int wg;         // threads per workgroup
    int rows_per_wg;
    int64_t grid;   // workgroups launched (grid-stride loops cover the rest)
    int chunks;     // split: chunks per row
    int64_t work;   // rows: row groups; split: M * chunks
};

// Tiles instantiated for the row kernel.
constexpr int kTeams[] = {4, 8, 16, 32, 64, 128, 256, 512, 1024};
constexpr int kVpls[] = {1, 2, 4, 8, 16};
constexpr int kMaxTeam = 1024;
constexpr int kMaxVpl = 16;
// Split-row chunk geometry.
constexpr int kSplitWG = 256;
constexpr int kSplitVPL = 4;

hipError_t launch_rows_f32(bool rms, const NormCall& c, const Plan& p);
hipError_t launch_rows_bf16(bool rms, const NormCall& c, const Plan& p);
hipError_t launch_rows_f16(bool rms, const NormCall& c, const Plan& p);
hipError_t launch_split_f32(bool rms, const NormCall& c, const Plan& p, float2* ws);
hipError_t launch_split_bf16(bool rms, const NormCall& c, const Plan& p, float2* ws);
hipError_t launch_split_f16(bool rms, const NormCall& c, const Plan& p, float2* ws);

}  // namespace mi355norm
