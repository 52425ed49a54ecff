// C ABI of libgdr: host-side validation and dispatch (declared in gdr.h).
//
// Every check runs on the host before anything is enqueued, so an error
// status means nothing was written.  No exception leaves this file.
#include "../../include/gdr.h"
#include "gdr_device.h"
#include "launch.h"

namespace gdr {

namespace {

__global__ void state_copy_kernel(const float* __restrict__ s0, float* __restrict__ s,
                                  int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        s[i] = s0 ? s0[i] : 0.f;
}

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dims_ok(int64_t dk, int64_t dv) {
    return (dk == 64 || dk == 128) && (dv == 64 || dv == 128);
}

bool dtype_ok(gdr_dtype_t d) { return d == GDR_F32 || d == GDR_BF16; }

bool flags_ok(uint32_t f) { return (f & ~GDR_L2NORM_QK) == 0; }

gdr_status_t from_hip(hipError_t e) { return e == hipSuccess ? GDR_OK : GDR_ERR_DEVICE; }

// Every listed pointer must be non-NULL and 16-byte aligned.
bool ptrs_ok(std::initializer_list<const void*> ps) {
    for (const void* p : ps)
        if (!p || !aligned(p)) return false;
    return true;
}

bool opt_ok(const void* p) { return !p || aligned(p); }

// Element-aligned pointer (scalar gates and outputs are accessed per element).
bool elem_ok(const void* p, size_t bytes) {
    return p && (reinterpret_cast<uintptr_t>(p) % bytes) == 0;
}

// Largest element count of any tensor must fit the kernels' 64-bit offsets.
bool sizes_ok(int64_t a, int64_t b, int64_t c) {
    if (a < 0 || b < 0 || c < 0) return false;
    const double n = (double)a * (double)b * (double)c;
    return n < 4.0e18;
}

// One work-item per element over n elements, 256 per workgroup, fits a
// dispatch (the backward's reductions).
bool grid_ok(int64_t n) { return n >= 0 && (n + 255) / 256 <= kMaxWorkItems / 256; }

// The per-head launches (the chunk kernels of both rules and both
// directions, the segment scans) run at most 2048 work-items per head
// (d_v = 128: the rule-2 forward's 4 row blocks x 512, the scans' 8 x 256)
// on a grid rounded up to 8 heads; BH heads must fit one dispatch.
bool heads_grid_ok(int64_t BH) { return BH >= 0 && (BH + 7) / 8 * 8 <= kMaxWorkItems / 2048; }

// The chunk kernels address one chunk of tokens (H heads x d channels each)
// with 32-bit byte offsets from a 64-bit chunk base.
bool heads_ok(int64_t H) { return H <= GDR_MAX_HEADS; }

}  // namespace

hipError_t launch_state_copy(const float* s0, float* s_final, int64_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(state_copy_kernel, dim3(stride_blocks(n)), dim3(256), 0, st, s0, s_final,
                       n);
    return hipGetLastError();
}

}  // namespace gdr

using namespace gdr;

static gdr_status_t chunk_common(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                 gdr_dtype_t in_dt, gdr_dtype_t out_dt, ChunkArgs& a) {
    if (B < 0 || T < 0 || H < 0 || Dk < 0 || Dv < 0) return GDR_ERR_INVALID;
    if (!sizes_ok(B, T, H) || !sizes_ok(B * T * H, Dk > Dv ? Dk : Dv, 1)) return GDR_ERR_INVALID;
    if (!heads_ok(H)) return GDR_ERR_INVALID;
    if (!dtype_ok(in_dt) || !dtype_ok(out_dt)) return GDR_ERR_UNSUPPORTED;
    if (!dims_ok(Dk, Dv)) return GDR_ERR_UNSUPPORTED;
    if (!heads_grid_ok(B * H)) return GDR_ERR_INVALID;
    a.B = B;
    a.T = T;
    a.H = H;
    a.Dk = Dk;
    a.Dv = Dv;
    a.in_bf16 = in_dt == GDR_BF16;
    a.out_bf16 = out_dt == GDR_BF16;
    return GDR_OK;
}

static gdr_status_t chunk_run(ChunkArgs& a) {
    if (a.B == 0 || a.H == 0) return GDR_OK;
    if (a.T == 0) {
        if (!a.s_final || a.s_final == a.s0) return GDR_OK;
        return from_hip(launch_state_copy(a.s0, a.s_final, a.B * a.H * a.Dv * a.Dk, a.stream));
    }
    hipError_t e;
    if (!a.in_bf16)
        e = launch_chunk_f32(a);
    else if (a.gated2)
        e = launch_gdr2_bf16(a);
    else
        e = launch_chunk_bf16(a);
    if (e == hipErrorNotSupported) return GDR_ERR_UNSUPPORTED;
    return from_hip(e);
}

extern "C" gdr_status_t gdr_chunk_fwd_ex(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                         int64_t Dv, gdr_dtype_t in_dt, const void* q,
                                         const void* k, const void* v, const float* alpha,
                                         const float* beta, const float* s0,
                                         gdr_dtype_t out_dt, void* o, float* s_final,
                                         uint32_t flags, hipStream_t stream) {
    if (!flags_ok(flags)) return GDR_ERR_UNSUPPORTED;
    ChunkArgs a{};
    gdr_status_t st = chunk_common(B, T, H, Dk, Dv, in_dt, out_dt, a);
    if (st != GDR_OK) return st;
    const bool empty = B == 0 || T == 0 || H == 0;
    if (!empty && (!ptrs_ok({q, k, v}) || !elem_ok(alpha, 4) || !elem_ok(beta, 4) ||
                   !elem_ok(o, out_dt == GDR_BF16 ? 2 : 4)))
        return GDR_ERR_INVALID;
    if (!opt_ok(s0) || !opt_ok(s_final)) return GDR_ERR_INVALID;
    a.gated2 = false;
    a.l2norm = (flags & GDR_L2NORM_QK) != 0;
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.beta = beta;
    a.s0 = s0;
    a.o = o;
    a.s_final = s_final;
    a.stream = stream;
    return chunk_run(a);
}

extern "C" gdr_status_t gdr_chunk_fwd(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                      int64_t Dv, gdr_dtype_t in_dt, const void* q,
                                      const void* k, const void* v, const float* alpha,
                                      const float* beta, const float* s0,
                                      gdr_dtype_t out_dt, void* o, float* s_final,
                                      hipStream_t stream) {
    return gdr_chunk_fwd_ex(B, T, H, Dk, Dv, in_dt, q, k, v, alpha, beta, s0, out_dt, o,
                            s_final, 0u, stream);
}

// Forward with the output gate fused on its stores.  bf16 inputs: one pass
// of the bf16 kernel writing y, the workspace holding the row blocks'
// exchange words; fp32 inputs: the vector-ALU forward into an fp32 o in the
// workspace, then the gate kernel.
extern "C" size_t gdr_chunk_fwd_gate_workspace_size(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                                    int64_t Dv, gdr_dtype_t in_dt) {
    if (B < 0 || T < 0 || H < 0 || !dims_ok(Dk, Dv) || !dtype_ok(in_dt)) return 0;
    if (!sizes_ok(B, T, H) || !sizes_ok(B * T * H, Dk > Dv ? Dk : Dv, 1)) return 0;
    if (!heads_ok(H)) return 0;
    if (B == 0 || T == 0 || H == 0) return 0;
    if (in_dt == GDR_BF16) return chunk_gate_xch_bytes(B, H, Dv);
    return (size_t)(B * T * H * Dv) * 4;
}

extern "C" gdr_status_t gdr_chunk_fwd_gate(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                           int64_t Dv, gdr_dtype_t in_dt, const void* q,
                                           const void* k, const void* v, const float* alpha,
                                           const float* beta, const float* s0,
                                           gdr_dtype_t g_dt, const void* g, const float* w,
                                           float eps, gdr_dtype_t out_dt, void* y,
                                           float* s_final, uint32_t flags, void* workspace,
                                           size_t workspace_bytes, hipStream_t stream) {
    if (!flags_ok(flags)) return GDR_ERR_UNSUPPORTED;
    ChunkArgs a{};
    gdr_status_t st = chunk_common(B, T, H, Dk, Dv, in_dt, out_dt, a);
    if (st != GDR_OK) return st;
    if (!dtype_ok(g_dt)) return GDR_ERR_UNSUPPORTED;
    if (!(eps >= 0.f) || eps > 3.0e38f) return GDR_ERR_INVALID;
    if (!opt_ok(s0) || !opt_ok(s_final) || !opt_ok(w)) return GDR_ERR_INVALID;
    if (T >= ((int64_t)1 << 36)) return GDR_ERR_INVALID;   // 32-bit chunk slots
    const bool empty = B == 0 || T == 0 || H == 0;
    if (!empty) {
        if (!ptrs_ok({q, k, v, g, y}) || !elem_ok(alpha, 4) || !elem_ok(beta, 4))
            return GDR_ERR_INVALID;
        const size_t need = gdr_chunk_fwd_gate_workspace_size(B, T, H, Dk, Dv, in_dt);
        if (!ptrs_ok({workspace}) || workspace_bytes < need) return GDR_ERR_INVALID;
    }
    a.gated2 = false;
    a.l2norm = (flags & GDR_L2NORM_QK) != 0;
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.beta = beta;
    a.s0 = s0;
    a.s_final = s_final;
    a.stream = stream;
    if (empty) {
        a.o = y;
        return chunk_run(a);   // no tokens: s_final gets s0 (or zeros)
    }
    if (a.in_bf16) {
        a.o = y;
        a.gate = g;
        a.gate_bf16 = g_dt == GDR_BF16;
        a.w = w;
        a.eps = eps;
        a.xch = workspace;
        const hipError_t e = launch_chunk_bf16_gate(a);
        if (e == hipErrorNotSupported) return GDR_ERR_UNSUPPORTED;
        return from_hip(e);
    }
    a.o = workspace;
    a.out_bf16 = false;
    if ((st = chunk_run(a)) != GDR_OK) return st;
    GateArgs ga;
    ga.N = B * T;
    ga.H = H;
    ga.Dv = Dv;
    ga.o_bf16 = false;
    ga.g_bf16 = g_dt == GDR_BF16;
    ga.out_bf16 = out_dt == GDR_BF16;
    ga.o = workspace;
    ga.g = g;
    ga.w = w;
    ga.eps = eps;
    ga.y = y;
    ga.stream = stream;
    return from_hip(launch_output_gate(ga));
}

// Sequence-split forward: workspace pieces, each rounded up to 256 bytes.
namespace {
struct SplitLayout {
    size_t R, P, Sin, vz, oP, total;
};
size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }
SplitLayout split_layout(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                         gdr_dtype_t in_dt, int64_t nseg, bool discard = false) {
    SplitLayout l{};
    const size_t bn = (size_t)(B * nseg * H);
    l.R = up256(bn * Dv * Dk * 4);
    l.P = up256(bn * Dk * Dk * 4);
    l.Sin = up256(bn * Dv * Dk * 4);
    // a zero v for the P pass: fp32 inputs only (the bf16 kernels take a
    // missing v as zero)
    l.vz = in_dt == GDR_BF16 ? 0 : up256((size_t)(B * T * H * Dk) * 4);
    // the P pass's output (and, with `discard`, the R pass's) when it
    // cannot go to o: bf16, max(Dk, Dv) columns; fp32 inputs only (the
    // bf16 kernels' state passes write no o)
    l.oP = in_dt == GDR_BF16 ? 0
           : discard         ? up256((size_t)(B * T * H * (Dk > Dv ? Dk : Dv)) * 2)
           : Dk == Dv        ? 0
                             : up256((size_t)(B * T * H * Dk) * 2);
    l.total = l.R + l.P + l.Sin + l.vz + l.oP;
    return l;
}
}  // namespace

// Passes 1-3 of the sequence split, on the segment batch `a` (B nseg
// segments of T / nseg tokens, inputs set): R (each segment from zero), P
// (v = 0 from the identity) and the scan into the start states Sin.  Only
// the passes' final states are wanted: the bf16 matrix-core kernels get
// o = NULL (the scalar-gate one then skips the output products, the
// channel-gate one its stores); the fp32 vector-ALU kernels write theirs to
// `o` (overwritten by the caller's last pass) or to the workspace's discard
// buffer when the layout has one.
static gdr_status_t split_states(const ChunkArgs& a, const SplitLayout& l, char* w, int64_t B,
                                 int64_t nseg, const float* s0, void* o) {
    float* R = reinterpret_cast<float*>(w);
    float* P = reinterpret_cast<float*>(w + l.R);
    float* Sin = reinterpret_cast<float*>(w + l.R + l.P);
    void* vz = w + l.R + l.P + l.Sin;
    void* oP = l.oP ? static_cast<void*>(w + l.R + l.P + l.Sin + l.vz) : o;
    const bool no_o = a.in_bf16;
    gdr_status_t st;
    // 1. each segment from a zero state: R
    ChunkArgs r = a;
    r.s0 = nullptr;
    r.o = no_o ? nullptr : l.oP && !o ? oP : o;
    r.out_bf16 = l.oP && !o ? true : a.out_bf16;
    r.s_final = R;
    if ((st = chunk_run(r)) != GDR_OK) return st;
    // 2. each segment with v = 0 from the identity: P (d_k x d_k).  The
    // bf16 kernels given no v (GDN-2: nor w) take v = 0 without reading
    // memory; the vector-ALU kernels read the zeroed buffer
    const bool v_null = a.in_bf16;
    hipError_t e = launch_identity(P, a.B * a.H, (int)a.Dk, a.stream);
    if (e == hipSuccess && !v_null) e = launch_zero(vz, (int64_t)l.vz, a.stream);
    if (e != hipSuccess) return GDR_ERR_DEVICE;
    ChunkArgs pa = a;
    pa.Dv = a.Dk;
    pa.v = v_null ? nullptr : vz;
    if (a.gated2) pa.write = pa.v;   // w (.) v = 0 either way; w needs Dk columns here
    pa.s0 = P;
    pa.s_final = P;
    pa.o = no_o ? nullptr : oP;
    pa.out_bf16 = l.oP ? true : a.out_bf16;
    if ((st = chunk_run(pa)) != GDR_OK) return st;
    // 3. segment start states
    SplitScanArgs sc{B, a.H, a.Dk, a.Dv, (int)nseg, s0, R, P, Sin, a.stream};
    return from_hip(launch_split_scan(sc));
}

extern "C" size_t gdr_chunk_fwd_split_workspace_size(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                                     int64_t Dv, gdr_dtype_t in_dt,
                                                     int64_t nseg) {
    if (B < 0 || T < 0 || H < 0 || nseg < 1 || nseg > (1 << 20)) return 0;
    if (!dims_ok(Dk, Dv) || !dtype_ok(in_dt)) return 0;
    if (!sizes_ok(B, T, H) || !sizes_ok(B * T * H, Dk > Dv ? Dk : Dv, 1)) return 0;
    if (!heads_ok(H)) return 0;
    if (!sizes_ok(B * nseg, H, 1)) return 0;
    if (nseg == 1 || T == 0 || B == 0 || H == 0) return 0;
    if (T % nseg != 0) return 0;
    return split_layout(B, T, H, Dk, Dv, in_dt, nseg).total;
}

// The split forward once the segment batch `a` (inputs, B nseg x T / nseg)
// is set and the common arguments are validated.
static gdr_status_t fwd_split_run(ChunkArgs& a, int64_t B, int64_t T, int64_t H, int64_t Dk,
                                  int64_t Dv, gdr_dtype_t in_dt, const float* s0, void* o,
                                  float* s_final, int64_t nseg, void* workspace,
                                  size_t workspace_bytes) {
    if (T % nseg != 0 || !sizes_ok(B * nseg, H, 1)) return GDR_ERR_INVALID;
    if (!heads_grid_ok(B * nseg * H)) return GDR_ERR_INVALID;
    if (!ptrs_ok({workspace}) || !opt_ok(s0) || !opt_ok(s_final)) return GDR_ERR_INVALID;
    const SplitLayout l = split_layout(B, T, H, Dk, Dv, in_dt, nseg);
    if (workspace_bytes < l.total) return GDR_ERR_INVALID;
    char* w = static_cast<char*>(workspace);
    float* Sin = reinterpret_cast<float*>(w + l.R + l.P);
    // the segments as a batch: [B, T, H, d] is [B nseg, T / nseg, H, d]
    a.B = B * nseg;
    a.T = T / nseg;
    gdr_status_t st;
    if ((st = split_states(a, l, w, B, nseg, s0, o)) != GDR_OK) return st;
    // 4. every segment from its start state: o, and the final states in place
    ChunkArgs f = a;
    f.s0 = Sin;
    f.s_final = Sin;
    f.o = o;
    if ((st = chunk_run(f)) != GDR_OK) return st;
    if (s_final)
        return from_hip(launch_seg_state(Sin, s_final, B, (int)nseg, (int)nseg - 1, H * Dv * Dk,
                                         a.stream));
    return GDR_OK;
}

extern "C" gdr_status_t gdr_chunk_fwd_split(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                            int64_t Dv, gdr_dtype_t in_dt, const void* q,
                                            const void* k, const void* v, const float* alpha,
                                            const float* beta, const float* s0,
                                            gdr_dtype_t out_dt, void* o, float* s_final,
                                            int64_t nseg, uint32_t flags, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream) {
    if (nseg < 1 || nseg > (1 << 20)) return GDR_ERR_INVALID;
    if (nseg == 1 || T == 0 || B == 0 || H == 0)
        return gdr_chunk_fwd_ex(B, T, H, Dk, Dv, in_dt, q, k, v, alpha, beta, s0, out_dt, o,
                                s_final, flags, stream);
    if (!flags_ok(flags)) return GDR_ERR_UNSUPPORTED;
    ChunkArgs a{};
    gdr_status_t st = chunk_common(B, T, H, Dk, Dv, in_dt, out_dt, a);
    if (st != GDR_OK) return st;
    if (!ptrs_ok({q, k, v}) || !elem_ok(alpha, 4) || !elem_ok(beta, 4) ||
        !elem_ok(o, out_dt == GDR_BF16 ? 2 : 4))
        return GDR_ERR_INVALID;
    a.gated2 = false;
    a.l2norm = (flags & GDR_L2NORM_QK) != 0;
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.beta = beta;
    a.stream = stream;
    return fwd_split_run(a, B, T, H, Dk, Dv, in_dt, s0, o, s_final, nseg, workspace,
                         workspace_bytes);
}

extern "C" gdr_status_t gdr2_chunk_fwd_split(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                             int64_t Dv, gdr_dtype_t in_dt, const void* q,
                                             const void* k, const void* v, const void* alpha,
                                             const void* erase, const void* write,
                                             const float* s0, gdr_dtype_t out_dt, void* o,
                                             float* s_final, int64_t nseg, uint32_t flags,
                                             void* workspace, size_t workspace_bytes,
                                             hipStream_t stream) {
    if (nseg < 1 || nseg > (1 << 20)) return GDR_ERR_INVALID;
    if (nseg == 1 || T == 0 || B == 0 || H == 0)
        return gdr2_chunk_fwd_ex(B, T, H, Dk, Dv, in_dt, q, k, v, alpha, erase, write, s0,
                                 out_dt, o, s_final, flags, stream);
    if (!flags_ok(flags)) return GDR_ERR_UNSUPPORTED;
    ChunkArgs a{};
    gdr_status_t st = chunk_common(B, T, H, Dk, Dv, in_dt, out_dt, a);
    if (st != GDR_OK) return st;
    if (!ptrs_ok({q, k, v, alpha, erase, write}) || !elem_ok(o, out_dt == GDR_BF16 ? 2 : 4))
        return GDR_ERR_INVALID;
    a.gated2 = true;
    a.l2norm = (flags & GDR_L2NORM_QK) != 0;
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.erase = erase;
    a.write = write;
    a.stream = stream;
    return fwd_split_run(a, B, T, H, Dk, Dv, in_dt, s0, o, s_final, nseg, workspace,
                         workspace_bytes);
}

// Sequence-split backward: the forward's split pieces, the segments' own
// contributions N and end gradients Gend, and the backward workspace of the
// segment batch.
namespace {
struct BwdSplitLayout {
    SplitLayout f;
    size_t N, G, bw, total;
};
BwdSplitLayout bwd_split_layout(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                gdr_dtype_t in_dt, int64_t nseg, bool gated2) {
    BwdSplitLayout l{};
    l.f = split_layout(B, T, H, Dk, Dv, in_dt, nseg, true);
    const size_t bn = (size_t)(B * nseg * H);
    l.N = up256(bn * Dv * Dk * 4);
    l.G = up256(bn * Dv * Dk * 4);
    l.bw = up256(gated2 ? bwd2_workspace_bytes(B * nseg, T / nseg, H, Dk, Dv)
                        : bwd_workspace_bytes(B * nseg, T / nseg, H, Dk, Dv));
    l.total = l.f.total + l.N + l.G + l.bw;
    return l;
}
}  // namespace

// The split backward once the segment batch `a` (forward inputs) is set and
// the arguments are validated.  run_bwd(s0, ds_final, ds0, workspace) runs
// the backward over the segment batch.
template <typename RunBwd>
static gdr_status_t bwd_split_run(ChunkArgs& a, const BwdSplitLayout& l, void* workspace,
                                  int64_t B, int64_t T, int64_t H, int64_t nseg, const float* s0,
                                  const float* ds_final, float* ds0, RunBwd run_bwd) {
    char* w = static_cast<char*>(workspace);
    float* P = reinterpret_cast<float*>(w + l.f.R);
    float* Sin = reinterpret_cast<float*>(w + l.f.R + l.f.P);
    float* N = reinterpret_cast<float*>(w + l.f.total);
    float* G = reinterpret_cast<float*>(w + l.f.total + l.N);
    void* bw = w + l.f.total + l.N + l.G;
    a.B = B * nseg;
    a.T = T / nseg;
    gdr_status_t st;
    // the segments' start states S_in and transitions P
    if ((st = split_states(a, l.f, w, B, nseg, s0, nullptr)) != GDR_OK) return st;
    // each segment's own contribution to dL/dS_in: its backward from a zero
    // end gradient (its other gradients are overwritten below)
    hipError_t e = run_bwd(Sin, nullptr, N, bw);
    if (e != hipSuccess) return GDR_ERR_DEVICE;
    // the segments' end gradients, last to first
    SplitScanArgs rs{B, H, a.Dk, a.Dv, (int)nseg, ds_final, N, P, G, a.stream};
    if ((e = launch_split_rscan(rs)) != hipSuccess) return GDR_ERR_DEVICE;
    // every segment from its start state with its end gradient
    if ((e = run_bwd(Sin, G, N, bw)) != hipSuccess) return GDR_ERR_DEVICE;
    if (ds0)
        return from_hip(launch_seg_state(N, ds0, B, (int)nseg, 0, H * a.Dv * a.Dk, a.stream));
    return GDR_OK;
}

static gdr_status_t bwd_split_check(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                    gdr_dtype_t in_dt, gdr_dtype_t dout_dt, int64_t nseg,
                                    uint32_t flags, ChunkArgs& a, uint32_t extra = 0u) {
    if (!flags_ok(flags & ~extra)) return GDR_ERR_UNSUPPORTED;
    gdr_status_t st = chunk_common(B, T, H, Dk, Dv, in_dt, GDR_BF16, a);
    if (st != GDR_OK) return st;
    if (!dtype_ok(dout_dt)) return GDR_ERR_UNSUPPORTED;
    if (T % nseg != 0 || !sizes_ok(B * nseg, H, 1)) return GDR_ERR_INVALID;
    if (!grid_ok(B * T * H * Dk) || !heads_grid_ok(B * nseg * H)) return GDR_ERR_INVALID;
    a.l2norm = (flags & GDR_L2NORM_QK) != 0;
    return GDR_OK;
}

extern "C" size_t gdr_chunk_bwd_split_workspace_size(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                                     int64_t Dv, gdr_dtype_t in_dt,
                                                     int64_t nseg) {
    if (nseg == 1 && dtype_ok(in_dt)) return gdr_chunk_bwd_workspace_size(B, T, H, Dk, Dv);
    if (gdr_chunk_fwd_split_workspace_size(B, T, H, Dk, Dv, in_dt, nseg) == 0) return 0;
    return bwd_split_layout(B, T, H, Dk, Dv, in_dt, nseg, false).total;
}

extern "C" size_t gdr2_chunk_bwd_split_workspace_size(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                                      int64_t Dv, gdr_dtype_t in_dt,
                                                      int64_t nseg) {
    if (nseg == 1 && dtype_ok(in_dt)) return gdr2_chunk_bwd_workspace_size(B, T, H, Dk, Dv);
    if (gdr_chunk_fwd_split_workspace_size(B, T, H, Dk, Dv, in_dt, nseg) == 0) return 0;
    // enough for the plain call too (GDR_SPLIT_FP32_STATES)
    const size_t split = bwd_split_layout(B, T, H, Dk, Dv, in_dt, nseg, true).total;
    const size_t plain = gdr2_chunk_bwd_workspace_size(B, T, H, Dk, Dv);
    return split > plain ? split : plain;
}

extern "C" gdr_status_t gdr_chunk_bwd_split(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                            int64_t Dv, gdr_dtype_t in_dt, const void* q,
                                            const void* k, const void* v, const float* alpha,
                                            const float* beta, const float* s0,
                                            gdr_dtype_t dout_dt, const void* dout,
                                            const float* ds_final, float* dq, float* dk,
                                            float* dv, float* dalpha, float* dbeta, float* ds0,
                                            int64_t nseg, uint32_t flags, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream) {
    if (nseg < 1 || nseg > (1 << 20)) return GDR_ERR_INVALID;
    if (nseg == 1 || T == 0 || B == 0 || H == 0)   // the plain call
        return gdr_chunk_bwd_ex(B, T, H, Dk, Dv, in_dt, q, k, v, alpha, beta, s0, dout_dt, dout,
                                ds_final, dq, dk, dv, dalpha, dbeta, ds0, workspace,
                                workspace_bytes, flags, stream);
    ChunkArgs a{};
    gdr_status_t st = bwd_split_check(B, T, H, Dk, Dv, in_dt, dout_dt, nseg, flags, a);
    if (st != GDR_OK) return st;
    if (!ptrs_ok({q, k, v, dout, dq, dk, dv, workspace}) || !elem_ok(alpha, 4) ||
        !elem_ok(beta, 4) || !elem_ok(dalpha, 4) || !elem_ok(dbeta, 4))
        return GDR_ERR_INVALID;
    if (!opt_ok(s0) || !opt_ok(ds_final) || !opt_ok(ds0)) return GDR_ERR_INVALID;
    const BwdSplitLayout l = bwd_split_layout(B, T, H, Dk, Dv, in_dt, nseg, false);
    if (workspace_bytes < l.total) return GDR_ERR_INVALID;
    a.gated2 = false;
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.beta = beta;
    a.stream = stream;
    BwdArgs b{};
    b.B = B * nseg;
    b.T = T / nseg;
    b.H = H;
    b.Dk = Dk;
    b.Dv = Dv;
    b.in_bf16 = in_dt == GDR_BF16;
    b.dout_bf16 = dout_dt == GDR_BF16;
    b.l2norm = a.l2norm;
    b.q = q;
    b.k = k;
    b.v = v;
    b.dout = dout;
    b.alpha = alpha;
    b.beta = beta;
    b.dq = dq;
    b.dk = dk;
    b.dv = dv;
    b.dalpha = dalpha;
    b.dbeta = dbeta;
    b.stream = stream;
    return bwd_split_run(a, l, workspace, B, T, H, nseg, s0, ds_final, ds0,
                         [&](const float* sin, const float* gend, float* d0, void* bw) {
                             b.s0 = sin;
                             b.ds_final = gend;
                             b.ds0 = d0;
                             b.workspace = bw;
                             return launch_chunk_bwd(b);
                         });
}

extern "C" gdr_status_t gdr2_chunk_bwd_split(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                             int64_t Dv, gdr_dtype_t in_dt, const void* q,
                                             const void* k, const void* v, const void* alpha,
                                             const void* erase, const void* write,
                                             const float* s0, gdr_dtype_t dout_dt,
                                             const void* dout, const float* ds_final, float* dq,
                                             float* dk, float* dv, float* dalpha, float* derase,
                                             float* dwrite, float* ds0, int64_t nseg,
                                             uint32_t flags, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream) {
    if (nseg < 1 || nseg > (1 << 20)) return GDR_ERR_INVALID;
    // one segment, or fp32 start states asked for: the plain call over the
    // whole sequence
    if (nseg == 1 || T == 0 || B == 0 || H == 0 || (flags & GDR_SPLIT_FP32_STATES))
        return gdr2_chunk_bwd_ex(B, T, H, Dk, Dv, in_dt, q, k, v, alpha, erase, write, s0,
                                 dout_dt, dout, ds_final, dq, dk, dv, dalpha, derase, dwrite, ds0,
                                 workspace, workspace_bytes, flags & ~GDR_SPLIT_FP32_STATES,
                                 stream);
    ChunkArgs a{};
    gdr_status_t st = bwd_split_check(B, T, H, Dk, Dv, in_dt, dout_dt, nseg, flags, a,
                                      GDR_SPLIT_FP32_STATES);
    if (st != GDR_OK) return st;
    if (!ptrs_ok({q, k, v, alpha, erase, write, dout, dq, dk, dv, dalpha, derase, dwrite,
                  workspace}))
        return GDR_ERR_INVALID;
    if (!opt_ok(s0) || !opt_ok(ds_final) || !opt_ok(ds0)) return GDR_ERR_INVALID;
    const BwdSplitLayout l = bwd_split_layout(B, T, H, Dk, Dv, in_dt, nseg, true);
    if (workspace_bytes < l.total) return GDR_ERR_INVALID;
    a.gated2 = true;
    // the start states from the matrix-core forward with every computed
    // operand split: the gradients inherit the states' error through S
    a.full = true;
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.erase = erase;
    a.write = write;
    a.stream = stream;
    Bwd2Args b{};
    b.B = B * nseg;
    b.T = T / nseg;
    b.H = H;
    b.Dk = Dk;
    b.Dv = Dv;
    b.in_bf16 = in_dt == GDR_BF16;
    b.dout_bf16 = dout_dt == GDR_BF16;
    b.l2norm = a.l2norm;
    b.q = q;
    b.k = k;
    b.v = v;
    b.alpha = alpha;
    b.erase = erase;
    b.write = write;
    b.dout = dout;
    b.dq = dq;
    b.dk = dk;
    b.dv = dv;
    b.dalpha = dalpha;
    b.derase = derase;
    b.dwrite = dwrite;
    b.stream = stream;
    return bwd_split_run(a, l, workspace, B, T, H, nseg, s0, ds_final, ds0,
                         [&](const float* sin, const float* gend, float* d0, void* bw) {
                             b.s0 = sin;
                             b.ds_final = gend;
                             b.ds0 = d0;
                             b.workspace = bw;
                             return launch_chunk2_bwd(b);
                         });
}

extern "C" gdr_status_t gdr2_chunk_fwd_ex(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                          int64_t Dv, gdr_dtype_t in_dt, const void* q,
                                          const void* k, const void* v, const void* alpha,
                                          const void* erase, const void* write,
                                          const float* s0, gdr_dtype_t out_dt, void* o,
                                          float* s_final, uint32_t flags, hipStream_t stream) {
    if (!flags_ok(flags)) return GDR_ERR_UNSUPPORTED;
    ChunkArgs a{};
    gdr_status_t st = chunk_common(B, T, H, Dk, Dv, in_dt, out_dt, a);
    if (st != GDR_OK) return st;
    const bool empty = B == 0 || T == 0 || H == 0;
    if (!empty && (!ptrs_ok({q, k, v, alpha, erase, write}) ||
                   !elem_ok(o, out_dt == GDR_BF16 ? 2 : 4)))
        return GDR_ERR_INVALID;
    if (!opt_ok(s0) || !opt_ok(s_final)) return GDR_ERR_INVALID;
    a.gated2 = true;
    a.l2norm = (flags & GDR_L2NORM_QK) != 0;
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.erase = erase;
    a.write = write;
    a.s0 = s0;
    a.o = o;
    a.s_final = s_final;
    a.stream = stream;
    return chunk_run(a);
}

extern "C" gdr_status_t gdr2_chunk_fwd(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                       int64_t Dv, gdr_dtype_t in_dt, const void* q,
                                       const void* k, const void* v, const void* alpha,
                                       const void* erase, const void* write,
                                       const float* s0, gdr_dtype_t out_dt, void* o,
                                       float* s_final, hipStream_t stream) {
    return gdr2_chunk_fwd_ex(B, T, H, Dk, Dv, in_dt, q, k, v, alpha, erase, write, s0, out_dt,
                             o, s_final, 0u, stream);
}

extern "C" gdr_status_t gdr_recurrent_step_ex(int64_t N, int64_t H, int64_t Dk, int64_t Dv,
                                              gdr_dtype_t in_dt, const void* q, const void* k,
                                              const void* v, const float* alpha,
                                              const float* beta, float* state,
                                              gdr_dtype_t out_dt, void* o, uint32_t flags,
                                              hipStream_t stream) {
    if (!flags_ok(flags)) return GDR_ERR_UNSUPPORTED;
    if (N < 0 || H < 0 || Dk < 0 || Dv < 0) return GDR_ERR_INVALID;
    // one 256-thread workgroup per (sequence, head)
    if (!sizes_ok(N, H, 1) || N * H > kMaxWorkItems / 256) return GDR_ERR_INVALID;
    if (!dtype_ok(in_dt) || !dtype_ok(out_dt)) return GDR_ERR_UNSUPPORTED;
    if (!dims_ok(Dk, Dv)) return GDR_ERR_UNSUPPORTED;
    if (N == 0 || H == 0) return GDR_OK;
    if (!ptrs_ok({q, k, v, state}) || !elem_ok(alpha, 4) || !elem_ok(beta, 4) ||
        !elem_ok(o, out_dt == GDR_BF16 ? 2 : 4))
        return GDR_ERR_INVALID;
    StepArgs a;
    a.N = N;
    a.H = H;
    a.Dk = Dk;
    a.Dv = Dv;
    a.in_bf16 = in_dt == GDR_BF16;
    a.out_bf16 = out_dt == GDR_BF16;
    a.l2norm = (flags & GDR_L2NORM_QK) != 0;
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.beta = beta;
    a.state = state;
    a.o = o;
    a.stream = stream;
    return from_hip(launch_step(a));
}

extern "C" gdr_status_t gdr_recurrent_step(int64_t N, int64_t H, int64_t Dk, int64_t Dv,
                                           gdr_dtype_t in_dt, const void* q, const void* k,
                                           const void* v, const float* alpha,
                                           const float* beta, float* state,
                                           gdr_dtype_t out_dt, void* o, hipStream_t stream) {
    return gdr_recurrent_step_ex(N, H, Dk, Dv, in_dt, q, k, v, alpha, beta, state, out_dt, o,
                                 0u, stream);
}

extern "C" gdr_status_t gdr_output_gate(int64_t N, int64_t H, int64_t Dv, gdr_dtype_t o_dt,
                                        const void* o, gdr_dtype_t g_dt, const void* g,
                                        const float* w, float eps, gdr_dtype_t out_dt, void* y,
                                        hipStream_t stream) {
    if (N < 0 || H < 0 || Dv < 0) return GDR_ERR_INVALID;
    if (!sizes_ok(N, H, Dv)) return GDR_ERR_INVALID;
    if (!dtype_ok(o_dt) || !dtype_ok(g_dt) || !dtype_ok(out_dt)) return GDR_ERR_UNSUPPORTED;
    if (Dv != 64 && Dv != 128) return GDR_ERR_UNSUPPORTED;
    if (!(eps >= 0.f) || eps > 3.0e38f) return GDR_ERR_INVALID;
    if (N == 0 || H == 0) return GDR_OK;
    if (!ptrs_ok({o, g, y}) || !opt_ok(w)) return GDR_ERR_INVALID;
    GateArgs a;
    a.N = N;
    a.H = H;
    a.Dv = Dv;
    a.o_bf16 = o_dt == GDR_BF16;
    a.g_bf16 = g_dt == GDR_BF16;
    a.out_bf16 = out_dt == GDR_BF16;
    a.o = o;
    a.g = g;
    a.w = w;
    a.eps = eps;
    a.y = y;
    a.stream = stream;
    return from_hip(launch_output_gate(a));
}

extern "C" size_t gdr_output_gate_bwd_workspace_size(int64_t N, int64_t H, int64_t Dv) {
    if (N < 0 || H < 0 || (Dv != 64 && Dv != 128) || !sizes_ok(N, H, Dv)) return 0;
    return gate_bwd_workspace_bytes(N * H, Dv);
}

// Checks shared by both gate backward calls; fills `a` except the workspace.
static gdr_status_t gate_bwd_check(int64_t N, int64_t H, int64_t Dv, gdr_dtype_t o_dt,
                                   const void* o, gdr_dtype_t g_dt, const void* g,
                                   const float* w, float eps, gdr_dtype_t dy_dt,
                                   const void* dy, float* dout, float* dg, float* dw,
                                   hipStream_t stream, GateBwdArgs& a) {
    if (N < 0 || H < 0 || Dv < 0) return GDR_ERR_INVALID;
    if (!sizes_ok(N, H, Dv)) return GDR_ERR_INVALID;
    if (!dtype_ok(o_dt) || !dtype_ok(g_dt) || !dtype_ok(dy_dt)) return GDR_ERR_UNSUPPORTED;
    if (Dv != 64 && Dv != 128) return GDR_ERR_UNSUPPORTED;
    if (!(eps >= 0.f) || eps > 3.0e38f) return GDR_ERR_INVALID;
    if (!opt_ok(w) || !opt_ok(dw)) return GDR_ERR_INVALID;
    if (N > 0 && H > 0 && !ptrs_ok({o, g, dy, dout, dg})) return GDR_ERR_INVALID;
    a.N = N;
    a.H = H;
    a.Dv = Dv;
    a.o_bf16 = o_dt == GDR_BF16;
    a.g_bf16 = g_dt == GDR_BF16;
    a.dy_bf16 = dy_dt == GDR_BF16;
    a.o = o;
    a.g = g;
    a.dy = dy;
    a.w = w;
    a.eps = eps;
    a.dout = dout;
    a.dg = dg;
    a.dw = dw;
    a.stream = stream;
    return GDR_OK;
}

extern "C" gdr_status_t gdr_output_gate_bwd(int64_t N, int64_t H, int64_t Dv, gdr_dtype_t o_dt,
                                            const void* o, gdr_dtype_t g_dt, const void* g,
                                            const float* w, float eps, gdr_dtype_t dy_dt,
                                            const void* dy, float* dout, float* dg, float* dw,
                                            void* workspace, size_t workspace_bytes,
                                            hipStream_t stream) {
    GateBwdArgs a{};
    gdr_status_t st = gate_bwd_check(N, H, Dv, o_dt, o, g_dt, g, w, eps, dy_dt, dy, dout, dg,
                                     dw, stream, a);
    if (st != GDR_OK) return st;
    if (N == 0 || H == 0) {
        // no rows: dw is zero
        if (dw) return from_hip(launch_state_copy(nullptr, dw, Dv, stream));
        return GDR_OK;
    }
    if (dw && (!ptrs_ok({workspace}) || workspace_bytes < gate_bwd_workspace_bytes(N * H, Dv)))
        return GDR_ERR_INVALID;
    a.workspace = workspace;
    return from_hip(launch_output_gate_bwd(a));
}

extern "C" gdr_status_t gdr_output_gate_bwd_noalloc(int64_t N, int64_t H, int64_t Dv,
                                                    gdr_dtype_t o_dt, const void* o,
                                                    gdr_dtype_t g_dt, const void* g,
                                                    const float* w, float eps,
                                                    gdr_dtype_t dy_dt, const void* dy,
                                                    float* dout, float* dg, float* dw,
                                                    hipStream_t stream) {
    GateBwdArgs a{};
    gdr_status_t st = gate_bwd_check(N, H, Dv, o_dt, o, g_dt, g, w, eps, dy_dt, dy, dout, dg,
                                     dw, stream, a);
    if (st != GDR_OK) return st;
    if (N == 0 || H == 0) {
        if (dw) return from_hip(launch_state_copy(nullptr, dw, Dv, stream));
        return GDR_OK;
    }
    if (dw) {
        // the partials go to the library's own array on the stream's device,
        // which must be the current device
        if (gate_bwd_workspace_bytes(N * H, Dv) > gate_bwd_scratch_bytes()) return GDR_ERR_INVALID;
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return GDR_ERR_DEVICE;
        if (stream) {
            hipDevice_t sdev = -1;
            if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return GDR_ERR_DEVICE;
            if (cur != (int)sdev) return GDR_ERR_INVALID;
        }
        float* p = nullptr;
        if (gate_bwd_scratch(&p) != hipSuccess) return GDR_ERR_DEVICE;
        a.workspace = p;
    }
    return from_hip(launch_output_gate_bwd(a));
}

extern "C" size_t gdr_chunk_bwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                               int64_t Dv) {
    if (B < 0 || T < 0 || H < 0 || !dims_ok(Dk, Dv)) return 0;
    if (!sizes_ok(B, T, H) || !sizes_ok(B * T * H, Dk > Dv ? Dk : Dv, 1)) return 0;
    if (!heads_ok(H)) return 0;
    return bwd_workspace_bytes(B, T, H, Dk, Dv);
}

extern "C" gdr_status_t gdr_chunk_bwd_ex(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                         int64_t Dv, gdr_dtype_t in_dt, const void* q,
                                         const void* k, const void* v, const float* alpha,
                                         const float* beta, const float* s0,
                                         gdr_dtype_t dout_dt, const void* dout,
                                         const float* ds_final, float* dq, float* dk, float* dv,
                                         float* dalpha, float* dbeta, float* ds0,
                                         void* workspace, size_t workspace_bytes, uint32_t flags,
                                         hipStream_t stream) {
    if (!flags_ok(flags)) return GDR_ERR_UNSUPPORTED;
    if (B < 0 || T < 0 || H < 0 || Dk < 0 || Dv < 0) return GDR_ERR_INVALID;
    if (!sizes_ok(B, T, H) || !sizes_ok(B * T * H, Dk > Dv ? Dk : Dv, 1)) return GDR_ERR_INVALID;
    if (!heads_ok(H)) return GDR_ERR_INVALID;
    if (!dtype_ok(in_dt) || !dtype_ok(dout_dt)) return GDR_ERR_UNSUPPORTED;
    if (!dims_ok(Dk, Dv)) return GDR_ERR_UNSUPPORTED;
    if (!heads_grid_ok(B * H)) return GDR_ERR_INVALID;
    if (!opt_ok(s0) || !opt_ok(ds_final) || !opt_ok(ds0)) return GDR_ERR_INVALID;
    if (B == 0 || H == 0) return GDR_OK;
    if (T == 0) {
        // no tokens: dS_0 = dS_T
        if (!ds0) return GDR_OK;
        return from_hip(launch_state_copy(ds_final, ds0, B * H * Dv * Dk, stream));
    }
    if (!ptrs_ok({q, k, v, dout, dq, dk, dv, workspace}) || !elem_ok(alpha, 4) ||
        !elem_ok(beta, 4) || !elem_ok(dalpha, 4) || !elem_ok(dbeta, 4))
        return GDR_ERR_INVALID;
    if (!grid_ok(B * T * H * Dk)) return GDR_ERR_INVALID;
    if (workspace_bytes < bwd_workspace_bytes(B, T, H, Dk, Dv)) return GDR_ERR_INVALID;
    BwdArgs a{};
    a.l2norm = (flags & GDR_L2NORM_QK) != 0;
    a.B = B;
    a.T = T;
    a.H = H;
    a.Dk = Dk;
    a.Dv = Dv;
    a.in_bf16 = in_dt == GDR_BF16;
    a.dout_bf16 = dout_dt == GDR_BF16;
    a.q = q;
    a.k = k;
    a.v = v;
    a.dout = dout;
    a.alpha = alpha;
    a.beta = beta;
    a.s0 = s0;
    a.ds_final = ds_final;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.dalpha = dalpha;
    a.dbeta = dbeta;
    a.ds0 = ds0;
    a.workspace = workspace;
    a.stream = stream;
    return from_hip(launch_chunk_bwd(a));
}

extern "C" gdr_status_t gdr_chunk_bwd(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                      gdr_dtype_t in_dt, const void* q, const void* k,
                                      const void* v, const float* alpha, const float* beta,
                                      const float* s0, gdr_dtype_t dout_dt, const void* dout,
                                      const float* ds_final, float* dq, float* dk, float* dv,
                                      float* dalpha, float* dbeta, float* ds0, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
    return gdr_chunk_bwd_ex(B, T, H, Dk, Dv, in_dt, q, k, v, alpha, beta, s0, dout_dt, dout,
                            ds_final, dq, dk, dv, dalpha, dbeta, ds0, workspace, workspace_bytes,
                            0u, stream);
}

extern "C" size_t gdr2_chunk_bwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                                int64_t Dv) {
    if (B < 0 || T < 0 || H < 0 || !dims_ok(Dk, Dv)) return 0;
    if (!sizes_ok(B, T, H) || !sizes_ok(B * T * H, Dk > Dv ? Dk : Dv, 1)) return 0;
    if (!heads_ok(H)) return 0;
    return bwd2_workspace_bytes(B, T, H, Dk, Dv);
}

extern "C" gdr_status_t gdr2_chunk_bwd_ex(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                          int64_t Dv, gdr_dtype_t in_dt, const void* q,
                                          const void* k, const void* v, const void* alpha,
                                          const void* erase, const void* write, const float* s0,
                                          gdr_dtype_t dout_dt, const void* dout,
                                          const float* ds_final, float* dq, float* dk, float* dv,
                                          float* dalpha, float* derase, float* dwrite,
                                          float* ds0, void* workspace, size_t workspace_bytes,
                                          uint32_t flags, hipStream_t stream) {
    if (!flags_ok(flags)) return GDR_ERR_UNSUPPORTED;
    if (B < 0 || T < 0 || H < 0 || Dk < 0 || Dv < 0) return GDR_ERR_INVALID;
    if (!sizes_ok(B, T, H) || !sizes_ok(B * T * H, Dk > Dv ? Dk : Dv, 1)) return GDR_ERR_INVALID;
    if (!heads_ok(H)) return GDR_ERR_INVALID;
    if (!dtype_ok(in_dt) || !dtype_ok(dout_dt)) return GDR_ERR_UNSUPPORTED;
    if (!dims_ok(Dk, Dv)) return GDR_ERR_UNSUPPORTED;
    if (!heads_grid_ok(B * H)) return GDR_ERR_INVALID;
    if (!opt_ok(s0) || !opt_ok(ds_final) || !opt_ok(ds0)) return GDR_ERR_INVALID;
    if (B == 0 || H == 0) return GDR_OK;
    if (T == 0) {
        if (!ds0) return GDR_OK;
        return from_hip(launch_state_copy(ds_final, ds0, B * H * Dv * Dk, stream));
    }
    if (!ptrs_ok({q, k, v, alpha, erase, write, dout, dq, dk, dv, dalpha, derase, dwrite,
                  workspace}))
        return GDR_ERR_INVALID;
    if (!grid_ok(B * T * H * Dk)) return GDR_ERR_INVALID;
    if (workspace_bytes < bwd2_workspace_bytes(B, T, H, Dk, Dv)) return GDR_ERR_INVALID;
    Bwd2Args a{};
    a.l2norm = (flags & GDR_L2NORM_QK) != 0;
    a.B = B;
    a.T = T;
    a.H = H;
    a.Dk = Dk;
    a.Dv = Dv;
    a.in_bf16 = in_dt == GDR_BF16;
    a.dout_bf16 = dout_dt == GDR_BF16;
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.erase = erase;
    a.write = write;
    a.dout = dout;
    a.s0 = s0;
    a.ds_final = ds_final;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.dalpha = dalpha;
    a.derase = derase;
    a.dwrite = dwrite;
    a.ds0 = ds0;
    a.workspace = workspace;
    a.stream = stream;
    return from_hip(launch_chunk2_bwd(a));
}

extern "C" gdr_status_t gdr2_chunk_bwd(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                       gdr_dtype_t in_dt, const void* q, const void* k,
                                       const void* v, const void* alpha, const void* erase,
                                       const void* write, const float* s0, gdr_dtype_t dout_dt,
                                       const void* dout, const float* ds_final, float* dq,
                                       float* dk, float* dv, float* dalpha, float* derase,
                                       float* dwrite, float* ds0, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
    return gdr2_chunk_bwd_ex(B, T, H, Dk, Dv, in_dt, q, k, v, alpha, erase, write, s0, dout_dt,
                             dout, ds_final, dq, dk, dv, dalpha, derase, dwrite, ds0, workspace,
                             workspace_bytes, 0u, stream);
}

extern "C" const char* gdr_status_string(gdr_status_t s) {
    switch (s) {
        case GDR_OK: return "ok";
        case GDR_ERR_INVALID: return "invalid argument (NULL or misaligned pointer, or bad size)";
        case GDR_ERR_UNSUPPORTED: return "unsupported head dims, dtype or flags";
        case GDR_ERR_DEVICE: return "HIP runtime error at launch";
    }
    return "unknown status";
}

extern "C" int gdr_version(void) { return 400; }
