// ss_kernels.h -- host-side launchers of the gfx950 selective-scan kernels.
// Called by the C ABI layer (ss_api.cpp) after it has validated every
// argument; the launchers only enqueue work and report launch errors.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssk {

struct ScanParams {
    int64_t batch, dim, seqlen;
    const void *u, *delta;
    const float *A;
    const void *B, *C;
    const float *D;
    const void *z;
    const float *bias;
    int softplus;
    const float *h0;
};

// chunk length of the checkpoints saved by the forward for the backward
constexpr int kCkptSpacing = 16;

struct FwdParams : ScanParams {
    void *out;
    float *last_state;
    float *ckpt;  // (batch, dim, ceil(L / 16), 16) or nullptr
};

struct BwdParams : ScanParams {
    const void *dout;
    const float *dlast;
    void *du, *ddelta;
    float *dA;
    void *dB, *dC;
    float *dD;
    void *dz;
    float *dbias;
    float *dh0;
    const float *ckpt;  // checkpoints saved by the forward, or nullptr
    void *workspace;
};

struct DecodeParams {
    int64_t batch, dim;
    float *state;
    const void *u, *delta;
    const float *A;
    const void *B, *C;
    const float *D;
    const void *z;
    const float *bias;
    int softplus;
    void *out;
};

// Records the next armed profiling event on `stream` (no-op when unarmed).
void profile_mark(hipStream_t stream);

hipError_t launch_fwd(const FwdParams &p, bool bf16, hipStream_t stream);
size_t bwd_workspace_bytes(int64_t batch, int64_t dim, int64_t seqlen);
hipError_t launch_bwd(const BwdParams &p, bool bf16, hipStream_t stream);
hipError_t launch_state_update(const DecodeParams &p, bool bf16, hipStream_t stream);

}  // namespace ssk
