// fa2_kernels.h -- host-side launch interface between the C ABI and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa2 {

// Block-sparse attention: the mask has one byte per block of kSparseBlock
// query rows x kSparseBlock keys, shared by every batch and head; the kernels
// compact a workgroup's mask row or column into an LDS list of tile indices,
// which bounds N.
constexpr int kSparseBlock = 128;
constexpr int kSparseMaxN = 262144;

struct FwdParams {
    const uint16_t* Q;  // bf16 (f16 in fa2_f16) [B, Hq, N, D]
    const uint16_t* K;  // bf16 [B, Hkv, N, D]
    const uint16_t* V;  // bf16 [B, Hkv, N, D]
    uint16_t* O;        // bf16 [B, Hq, N, D]
    uint16_t* Olo;      // bf16 [B, Hq, N, D]: O's rounding residual (NULL: not written)
    float* L;           // fp32 [B, Hq, N]
    int B, Hq, Hkv, N, G;
    int n_qtiles;       // ceil(N / rows per workgroup)
    float c;            // scale * log2(e): scores enter exp2 in the log2 domain
    const uint8_t* bmask;  // block-sparse mask [nb, nb] (NULL: dense attention)
    int nb;                // ceil(N / kSparseBlock)
};

struct BwdParams {
    const uint16_t* Q;
    const uint16_t* K;
    const uint16_t* V;
    const uint16_t* O;
    const uint16_t* Olo;  // O's rounding residual, added to O in D (NULL: D from O alone)
    const float* L;
    const uint16_t* dO;
    uint16_t* dQ;
    uint16_t* dK;
    uint16_t* dV;
    float* Dneg;   // fp32 [B, Hq, Npad]  workspace: -D = -rowsum(dO o (O + Olo)); 0 past N
    float* L2;     // fp32 [B, Hq, Npad]  workspace: L * log2(e); +inf past N (P = 0 there)
    float* dQacc;  // fp32 [B, Hq, N, D]  workspace: dQ accumulated with atomics
    int B, Hq, Hkv, N, G;
    int Npad;      // N rounded up to a multiple of kBwdRowPad
    float scale;
    float c;       // scale * log2(e)
    const uint8_t* bmask;  // block-sparse mask [nb, nb] (NULL: dense attention)
    int nb;                // ceil(N / kSparseBlock)
};

// Row padding of the backward's per-row workspace arrays (one query tile of
// the K/V-tile loop), so that whole tiles of L and D can be copied unchecked.
constexpr int kBwdRowPad = 64;

hipError_t launch_fwd(const FwdParams& p, int d, bool causal, hipStream_t stream);
// stages: bit 0 preprocess (D; zeroes the dQ accumulator in atomic mode), bit 1 the K/V-tile
// loop (dK, dV; plus dQ atomics in atomic mode), bit 2 dQ (its own pass, or the
// accumulator's conversion in atomic mode); bit 3 selects atomic mode.
hipError_t launch_bwd(const BwdParams& p, int d, bool causal, unsigned stages, hipStream_t stream);

}  // namespace fa2

// The same kernels compiled for f16 elements (the kernel sources built with
// FA2_F16=1); the parameter blocks are shared, their 16-bit pointers then hold f16.
namespace fa2_f16 {
using fa2::BwdParams;
using fa2::FwdParams;
using fa2::kBwdRowPad;
using fa2::kSparseBlock;
using fa2::kSparseMaxN;
hipError_t launch_fwd(const FwdParams& p, int d, bool causal, hipStream_t stream);
hipError_t launch_bwd(const BwdParams& p, int d, bool causal, unsigned stages, hipStream_t stream);
}  // namespace fa2_f16
