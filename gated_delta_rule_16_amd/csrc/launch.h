// Internal launch interface between the C ABI (gdr_api.cpp) and the kernels.
// Arguments arrive here already validated: dims in {64, 128}, sizes > 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

struct StepArgs {
    int64_t N, H, Dk, Dv;
    bool in_bf16, out_bf16;
    bool l2norm;            // normalise q, k on load (GDR_L2NORM_QK)
    const void *q, *k, *v;
    const float *alpha, *beta;
    float* state;
    void* o;
    hipStream_t stream;
};

// One struct for both chunked rules.  For the scalar-gated rule alpha and
// beta are fp32 [B,T,H] and erase/write are unused; for Gated Delta Rule-2
// alpha, erase ([B,T,H,Dk]) and write ([B,T,H,Dv]) are in the input dtype
// and beta is unused.
struct ChunkArgs {
    int64_t B, T, H, Dk, Dv;
    bool in_bf16, out_bf16;
    bool gated2;
    bool l2norm;            // normalise q, k on load (GDR_L2NORM_QK)
    bool full;              // rule 2, bf16 inputs: every computed operand split
    const void *q, *k, *v;
    const void *alpha, *beta, *erase, *write;
    const float* s0;
    void* o;                // NULL: no o (bf16 matrix-core kernels only)
    float* s_final;
    hipStream_t stream;
    // output gate fused on the stores of the bf16 scalar-gate kernel
    // (gdr_chunk_fwd_gate): o receives y; gate [B,T,H,Dv], w [Dv] or NULL,
    // xch the row blocks' exchange words (chunk_gate_xch_bytes)
    const void* gate;
    bool gate_bf16;
    const float* w;
    float eps;
    void* xch;
};

// Output gate: o, g [N, H, Dv]; w [Dv] fp32 or NULL.
struct GateArgs {
    int64_t N, H, Dv;
    bool o_bf16, g_bf16, out_bf16;
    const void *o, *g;
    const float* w;
    float eps;
    void* y;
    hipStream_t stream;
};

// Backward of the output gate: o, g, dy [N, H, Dv]; dout, dg fp32; dw [Dv]
// fp32 or NULL (then no workspace).
struct GateBwdArgs {
    int64_t N, H, Dv;
    bool o_bf16, g_bf16, dy_bf16;
    const void *o, *g, *dy;
    const float* w;
    float eps;
    float *dout, *dg, *dw;
    void* workspace;
    hipStream_t stream;
};

// Backward of the scalar-gate rule; gradients fp32, workspace from the caller.
struct BwdArgs {
    int64_t B, T, H, Dk, Dv;
    bool in_bf16, dout_bf16;
    bool l2norm;            // q, k normalised on load (GDR_L2NORM_QK)
    const void *q, *k, *v, *dout;
    const float *alpha, *beta, *s0, *ds_final;
    float *dq, *dk, *dv, *dalpha, *dbeta, *ds0;
    void* workspace;
    hipStream_t stream;
};

// Backward of Gated Delta Rule-2: alpha, erase [B,T,H,Dk] and write [B,T,H,Dv]
// in the input dtype; gradients fp32 with the inputs' shapes.
struct Bwd2Args {
    int64_t B, T, H, Dk, Dv;
    bool in_bf16, dout_bf16;
    bool l2norm;            // q, k normalised on load (GDR_L2NORM_QK)
    const void *q, *k, *v, *alpha, *erase, *write, *dout;
    const float *s0, *ds_final;
    float *dq, *dk, *dv, *dalpha, *derase, *dwrite, *ds0;
    void* workspace;
    hipStream_t stream;
};

// Scan over segment transitions (sequence-split forward).  States are
// [B nseg, H, Dv, Dk]; P is [B nseg, H, Dk, Dk]; s0 [B, H, Dv, Dk] or NULL.
struct SplitScanArgs {
    int64_t B, H, Dk, Dv;
    int nseg;
    const float *s0, *R, *P;
    float* Sin;
    hipStream_t stream;
};

// An HSA dispatch covers at most 2^32 - 1 work-items in each grid dimension
// (workgroups x workgroup size); every launch here is one-dimensional.
constexpr int64_t kMaxWorkItems = 0xffffffffLL;

// Workgroups of a grid-stride elementwise launch over n items, 256 threads
// each: enough to fill the chip, never past the work-item limit.
inline unsigned stride_blocks(int64_t n) {
    const int64_t b = (n + 255) / 256;
    return (unsigned)(b < 16384 ? b : 16384);
}

hipError_t launch_step(const StepArgs& a);
hipError_t launch_identity(float* x, int64_t n, int d, hipStream_t st);
hipError_t launch_zero(void* x, int64_t bytes, hipStream_t st);
hipError_t launch_split_scan(const SplitScanArgs& a);
hipError_t launch_split_rscan(const SplitScanArgs& a);
hipError_t launch_seg_state(const float* F, float* sf, int64_t B, int nseg, int seg,
                            int64_t per, hipStream_t st);
hipError_t launch_chunk_bwd(const BwdArgs& a);
size_t bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv);
hipError_t launch_chunk2_bwd(const Bwd2Args& a);
size_t bwd2_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv);
hipError_t launch_output_gate(const GateArgs& a);
hipError_t launch_output_gate_bwd(const GateBwdArgs& a);
size_t gate_bwd_workspace_bytes(int64_t rows, int64_t Dv);
// The library's own dw-partials array for gdr_output_gate_bwd_noalloc: its
// size in bytes, and its device address on the current device.
size_t gate_bwd_scratch_bytes();
hipError_t gate_bwd_scratch(float** out);
// fp32 inputs: VALU kernels, both rules.
hipError_t launch_chunk_f32(const ChunkArgs& a);
// bf16 inputs, scalar gates: bf16 MFMA kernel.
hipError_t launch_chunk_bf16(const ChunkArgs& a);
// The same with the output gate fused on its stores (zeroes a.xch first).
hipError_t launch_chunk_bf16_gate(const ChunkArgs& a);
size_t chunk_gate_xch_bytes(int64_t B, int64_t H, int64_t Dv);
// bf16 inputs, channel gates: bf16 MFMA kernel.
hipError_t launch_gdr2_bf16(const ChunkArgs& a);
// Copy s0 (or zeros) into s_final for an empty sequence.
hipError_t launch_state_copy(const float* s0, float* s_final, int64_t n, hipStream_t st);

}  // namespace gdr
