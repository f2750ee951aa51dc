// C-ABI entry points of libssm, the chunk-carry combine and the empty-sequence fill.
//
// Long sequences are cut into chunks: a carry pass stores, per chunk and state,
// the chunk's decay P (the product of A_bar over the chunk: exp(A sum delta)
// for the exponential discretisations) and the end state H from h = 0; the
// combine folds them in order with (P1, H1) o (P2, H2) = (P2 P1, P2 H1 + H2) (skill page
// "State Space Models Mamba", section "Hardware-Efficient Scan": the
// recurrence is linear, so it admits an associative scan); a second scan pass
// then starts every chunk from its carried-in state.
#include "ssm_device.h"

#include <mutex>

namespace ssm {
namespace {

// Fold chunk carries in sequence order, one thread per (b, d, n):
//   h_in(0) = h0,  h_in(c+1) = P_c * h_in(c) + H_c
// and overwrite slot c with h_in(c+1), the state chunk c+1 starts from.
__global__ void __launch_bounds__(256) combine_kernel(ScanArgs a) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t D = a.D, N = a.N;
    if (i >= a.B * D * N) return;
    const int64_t dn = i % (D * N);
    const int64_t b = i / (N * D);
    float h = a.h0 ? a.h0[i] : 0.0f;
    const int64_t C1 = a.n_chunks - 1;
    for (int64_t c = 0; c < C1; ++c) {
        const int64_t at = (b * C1 + c) * D * N + dn;
        h = __builtin_fmaf(a.ws_P[at], h, a.ws_H[at]);
        a.ws_H[at] = h;
    }
}

// n 16-bit words of zeros (any output of a gradient that has no terms)
__global__ void __launch_bounds__(256) zero16_kernel(uint16_t *p, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

// h_last = h0 (or zeros) for an empty sequence.
__global__ void __launch_bounds__(256) fill_state_kernel(float *h_last, const float *h0, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) h_last[i] = h0 ? h0[i] : 0.0f;
}


int hip_fail(const char *what, hipError_t e) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return SSM_EHIP;
}

hipError_t launch_scan_any(const ScanArgs &a, dim3 grid, const ScanPlan &p, int disc, bool bf16,
                           bool has_z, bool carry, hipStream_t s) {
    if (p.fast) {
        if (disc == kZOH) return launch_scan_fast_zoh(a, grid, p, bf16, has_z, carry, s);
        if (disc == kBilinear) return launch_scan_fast_bilinear(a, grid, p, bf16, has_z, carry, s);
        return launch_scan_fast_mamba(a, grid, p, bf16, has_z, carry, s);
    }
    if (disc == kZOH) return launch_scan_generic_zoh(a, grid, p, bf16, has_z, carry, s);
    if (disc == kBilinear) return launch_scan_generic_bilinear(a, grid, p, bf16, has_z, carry, s);
    return launch_scan_generic_mamba(a, grid, p, bf16, has_z, carry, s);
}

}  // namespace
}  // namespace ssm

namespace ssm {
namespace {

// The forward on a checked plan: B/C pre-pass, chunk carries and their combine (several
// chunks), then every chunk from its carried-in state producing y (and, given ckpt, the
// state before every 8th step, for the backward).
int run_scan(const ScanPlan &p, int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
             const void *x, const void *delta, const float *A, const void *B, const void *C,
             const float *Dskip, const void *z, const float *h0, float *h_last, void *y,
             int delta_softplus, const ssm_variant *variant, void *workspace, float *ckpt,
             int64_t ck_nblk, hipStream_t s) {
    ScanArgs a;
    a.B = batch; a.L = seqlen; a.D = dim; a.N = dstate;
    a.x = x; a.delta = delta; a.z = z; a.Bm = B; a.Cm = C;
    a.A = A; a.Dskip = Dskip; a.h0 = h0; a.h_last = h_last; a.y = y;
    a.softplus = delta_softplus;
    a.dbias = variant_bias(variant);
    const int disc = variant_disc(variant);
    a.structured = p.structured ? 1 : 0;
    a.NW = p.NW;
    a.chunk_len = p.chunk_len;
    a.n_chunks = p.n_chunks;
    a.ws_P = p.n_chunks > 1 ? reinterpret_cast<float *>(static_cast<char *>(workspace) + p.ws_P_off) : nullptr;
    a.ws_H = p.n_chunks > 1 ? reinterpret_cast<float *>(static_cast<char *>(workspace) + p.ws_H_off) : nullptr;
    a.ws_BC = p.fast ? reinterpret_cast<float *>(static_cast<char *>(workspace) + p.ws_BC_off) : nullptr;
    a.bc_lpad = p.bc_lpad;
    const unsigned dblocks = static_cast<unsigned>((dim + kChannelsPerBlock - 1) / kChannelsPerBlock);
    const bool bf16 = dtype == SSM_DTYPE_BF16;
    const bool has_z = z != nullptr;
    hipError_t e;
    if (p.fast) {
        // 0) B/C rows of every chunk to fp32, interleaved per state group, zero-padded
        e = launch_bc_pack(a, p, disc, bf16, s);
        if (e != hipSuccess) return hip_fail("B/C pack launch", e);
    }
    if (p.n_chunks > 1) {
        // 1) carries of every chunk but the last
        dim3 g1(dblocks, static_cast<unsigned>(batch), static_cast<unsigned>(p.n_chunks - 1));
        e = launch_scan_any(a, g1, p, disc, bf16, false, true, s);
        if (e != hipSuccess) return hip_fail("scan carry launch", e);
        // 2) fold the carries in order
        const int64_t n = batch * dim * dstate;
        hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, a);
        e = hipGetLastError();
        if (e != hipSuccess) return hip_fail("carry combine launch", e);
    }
    // 3) every chunk from its carried-in state, producing y (and the checkpoints)
    dim3 g3(dblocks, static_cast<unsigned>(batch), static_cast<unsigned>(p.n_chunks));
    a.ckpt = ckpt;
    a.ck_nblk = ck_nblk;
    e = ckpt ? launch_scan_save(a, g3, p, disc, bf16, has_z, s) : launch_scan_any(a, g3, p, disc, bf16, has_z, false, s);
    if (e != hipSuccess) return hip_fail("scan launch", e);
    return SSM_OK;
}

}  // namespace
}  // namespace ssm

extern "C" int ssm_scan_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                            const void *x, const void *delta, const float *A, const void *B,
                            const void *C, const float *Dskip, const void *z, const float *h0,
                            float *h_last, void *y, int delta_softplus, const ssm_variant *variant,
                            const ssm_scan_opts *opts, void *workspace, size_t workspace_bytes,
                            void *stream) {
    using namespace ssm;
    clear_error();
    ScanPlan p;
    int st = check_scan(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, Dskip, z, h0, h_last,
                        y, delta_softplus, variant, opts, workspace, workspace_bytes, &p);
    if (st != SSM_OK) return st;
    if (batch == 0 || dim == 0) return SSM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (seqlen == 0) {
        if (!h_last) return SSM_OK;
        const int64_t n = batch * dim * dstate;
        hipLaunchKernelGGL(fill_state_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                           0, s, h_last, h0, n);
        hipError_t e = hipGetLastError();
        return e == hipSuccess ? SSM_OK : hip_fail("fill_state launch", e);
    }
    return run_scan(p, batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, Dskip, z, h0, h_last, y,
                    delta_softplus, variant, workspace, nullptr, 0, s);
}

// ---- the forward for callers that cannot allocate: its workspace is a fixed device array

namespace ssm {
namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;   // SSM_NOALLOC_SCRATCH_BYTES
constexpr int kMaxDevices = 64;
// One copy per GPU, held from the library's load until the process ends.  In host code this
// name is not a device address: host code uses the per-device address from
// hipGetSymbolAddress (scratch_ptr) wherever it needs the array's memory.
__device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The scratch array's address on the current device (looked up once per device).
int scratch_ptr(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    if (dev < 0 || dev >= kMaxDevices) {
        set_error("device %d is beyond the %d devices the fixed scratch supports", dev, kMaxDevices);
        return SSM_EUNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail("hipGetSymbolAddress(scratch)", e);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SSM_OK;
}
}  // namespace
}  // namespace ssm

extern "C" size_t ssm_noalloc_scratch_bytes(void) { return ssm::kScratchBytes; }

extern "C" int ssm_scan_fwd_noalloc(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                                    const void *x, const void *delta, const float *A, const void *B,
                                    const void *C, const float *Dskip, const void *z, const float *h0,
                                    float *h_last, void *y, int delta_softplus, const ssm_variant *variant,
                                    const ssm_scan_opts *opts, void *stream) {
    using namespace ssm;
    clear_error();
    ScanPlan p;
    int st = plan_scan(batch, seqlen, dim, dstate, dtype, opts, &p);
    if (st != SSM_OK) return st;
    if (p.ws_bytes > kScratchBytes) {
        set_error("this shape needs %zu bytes of workspace; the fixed scratch holds %zu (use ssm_scan_fwd "
                  "with a caller-allocated workspace)", p.ws_bytes, kScratchBytes);
        return SSM_EWORKSPACE;
    }
    void *ws = nullptr;
    if (p.ws_bytes > 0 && batch > 0 && dim > 0 && seqlen > 0) {
        st = scratch_ptr(&ws);
        if (st != SSM_OK) return st;
    }
    st = check_scan(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, Dskip, z, h0, h_last, y,
                    delta_softplus, variant, opts, ws, ws ? kScratchBytes : 0, &p);
    if (st != SSM_OK) return st;
    if (batch == 0 || dim == 0) return SSM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (seqlen == 0) {
        if (!h_last) return SSM_OK;
        const int64_t n = batch * dim * dstate;
        hipLaunchKernelGGL(fill_state_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                           0, s, h_last, h0, n);
        hipError_t e = hipGetLastError();
        return e == hipSuccess ? SSM_OK : hip_fail("fill_state launch", e);
    }
    return run_scan(p, batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, Dskip, z, h0, h_last, y,
                    delta_softplus, variant, ws, nullptr, 0, s);
}

extern "C" int ssm_state_update(int64_t batch, int64_t dim, int64_t dstate, int dtype, float *h,
                                const void *x, const void *delta, const float *A, const void *B,
                                const void *C, const float *Dskip, const void *z, void *y,
                                int delta_softplus, const ssm_variant *variant, void *stream) {
    using namespace ssm;
    clear_error();
    int st = check_state_update(batch, dim, dstate, dtype, h, x, delta, A, B, C, Dskip, z, y,
                                delta_softplus, variant);
    if (st != SSM_OK) return st;
    if (batch == 0 || dim == 0) return SSM_OK;
    UpdArgs a;
    a.B = batch; a.D = dim; a.N = dstate; a.h = h;
    a.x = x; a.delta = delta; a.z = z; a.Bm = B; a.Cm = C; a.A = A; a.Dskip = Dskip; a.y = y;
    a.softplus = delta_softplus;
    a.dbias = variant_bias(variant);
    const int G = (dstate % 4 == 0) ? 4 : 1;
    int lpc = 1;
    while (lpc * G < dstate) lpc *= 2;
    a.lpc = lpc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_state_update(a, variant_disc(variant), dtype == SSM_DTYPE_BF16, z != nullptr, s);
    return e == hipSuccess ? SSM_OK : hip_fail("state update launch", e);
}

extern "C" int ssm_scan_fwd_save(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                                 const void *x, const void *delta, const float *A, const void *B,
                                 const void *C, const float *Dskip, const void *z, const float *h0,
                                 float *h_last, void *y, int delta_softplus, const ssm_variant *variant,
                                 float *checkpoints, void *workspace, size_t workspace_bytes, void *stream) {
    using namespace ssm;
    clear_error();
    BwdPlan bp;
    int st = check_scan_save(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, Dskip, z, h0, h_last, y,
                             delta_softplus, variant, checkpoints, workspace, workspace_bytes, &bp);
    if (st != SSM_OK) return st;
    if (batch == 0 || dim == 0) return SSM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (seqlen == 0) {   // no steps and no checkpoints: h_last = h0
        if (!h_last) return SSM_OK;
        const int64_t n = batch * dim * dstate;
        hipLaunchKernelGGL(fill_state_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                           0, s, h_last, h0, n);
        hipError_t e = hipGetLastError();
        return e == hipSuccess ? SSM_OK : hip_fail("fill_state launch", e);
    }
    return run_scan(bp.fwd, batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, Dskip, z, h0, h_last, y,
                    delta_softplus, variant, workspace, checkpoints, bp.nblk, s);
}

extern "C" int ssm_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                            const void *x, const void *delta, const float *A, const void *B,
                            const void *C, const float *Dskip, const void *z, const float *h0,
                            const void *dy, const float *dh_last, void *dx, void *ddelta, float *dA,
                            void *dB, void *dC, float *dD, void *dz, float *dh0, int delta_softplus,
                            int discretization, const float *delta_bias, float *ddelta_bias,
                            const float *checkpoints, void *workspace, size_t workspace_bytes,
                            void *stream) {
    using namespace ssm;
    clear_error();
    BwdPlan p;
    int st = check_scan_bwd(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, Dskip, z, h0, dy,
                            dh_last, dx, ddelta, dA, dB, dC, dD, dz, dh0, delta_softplus, discretization,
                            delta_bias, ddelta_bias, checkpoints, workspace, workspace_bytes, &p);
    if (st != SSM_OK) return st;
    if (batch == 0 || dim == 0) return SSM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (seqlen == 0) {
        // no steps: dh0 = dh_last, and the reductions over steps are zero
        if (dh0) {
            const int64_t n = batch * dim * dstate;
            hipLaunchKernelGGL(fill_state_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                               0, s, dh0, dh_last, n);
            e = hipGetLastError();
            if (e != hipSuccess) return hip_fail("fill_state launch", e);
        }
        hipLaunchKernelGGL(fill_state_kernel, dim3(static_cast<unsigned>((dim * dstate + 255) / 256)),
                           dim3(256), 0, s, dA, static_cast<const float *>(nullptr), dim * dstate);
        e = hipGetLastError();
        if (e != hipSuccess) return hip_fail("fill_state launch", e);
        if (Dskip && dD) {
            hipLaunchKernelGGL(fill_state_kernel, dim3(static_cast<unsigned>((dim + 255) / 256)), dim3(256),
                               0, s, dD, static_cast<const float *>(nullptr), dim);
            e = hipGetLastError();
            if (e != hipSuccess) return hip_fail("fill_state launch", e);
        }
        if (delta_bias) {
            hipLaunchKernelGGL(fill_state_kernel, dim3(static_cast<unsigned>((dim + 255) / 256)), dim3(256),
                               0, s, ddelta_bias, static_cast<const float *>(nullptr), dim);
            e = hipGetLastError();
            if (e != hipSuccess) return hip_fail("fill_state launch", e);
        }
        return SSM_OK;
    }
    char *ws = static_cast<char *>(workspace);
    const bool bf16 = dtype == SSM_DTYPE_BF16;
    // 1) checkpoints: the specialised forward kernel over the sequence, storing the state
    //    before every 8th step (B/C packed first, as for the forward); with several chunks
    //    the forward's carries and combine come first, and every chunk starts from its
    //    carried-in state.  Skipped when the caller passes the checkpoints that
    //    ssm_scan_fwd_save stored.
    if (!checkpoints) {
        char *fws = ws + p.fwd_off;
        ScanArgs fa;
        fa.B = batch; fa.L = seqlen; fa.D = dim; fa.N = dstate;
        fa.x = x; fa.delta = delta; fa.z = nullptr; fa.Bm = B; fa.Cm = C;
        fa.A = A; fa.Dskip = nullptr; fa.h0 = h0; fa.h_last = nullptr; fa.y = nullptr;
        fa.softplus = delta_softplus;
        fa.dbias = delta_bias;
        fa.structured = p.fwd.structured ? 1 : 0;
        fa.NW = p.fwd.NW;
        fa.chunk_len = p.fwd.chunk_len;
        fa.n_chunks = p.fwd.n_chunks;
        fa.ws_P = p.fwd.n_chunks > 1 ? reinterpret_cast<float *>(fws + p.fwd.ws_P_off) : nullptr;
        fa.ws_H = p.fwd.n_chunks > 1 ? reinterpret_cast<float *>(fws + p.fwd.ws_H_off) : nullptr;
        fa.ws_BC = reinterpret_cast<float *>(fws + p.fwd.ws_BC_off);
        fa.bc_lpad = p.fwd.bc_lpad;
        fa.ckpt = reinterpret_cast<float *>(ws + p.ckpt_off);
        fa.ck_nblk = p.nblk;
        e = launch_bc_pack(fa, p.fwd, discretization, bf16, s);
        if (e != hipSuccess) return hip_fail("B/C pack launch", e);
        const unsigned dblocks = static_cast<unsigned>(dim / 64);
        if (p.fwd.n_chunks > 1) {
            dim3 g1(dblocks, static_cast<unsigned>(batch), static_cast<unsigned>(p.fwd.n_chunks - 1));
            e = launch_scan_any(fa, g1, p.fwd, discretization, bf16, false, true, s);
            if (e != hipSuccess) return hip_fail("checkpoint carry launch", e);
            const int64_t n = batch * dim * dstate;
            hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, fa);
            e = hipGetLastError();
            if (e != hipSuccess) return hip_fail("checkpoint carry combine launch", e);
        }
        e = launch_scan_ckpt(fa, dim3(dblocks, static_cast<unsigned>(batch), static_cast<unsigned>(p.fwd.n_chunks)),
                             p.fwd, discretization, bf16, s);
        if (e != hipSuccess) return hip_fail("checkpoint pass launch", e);
    }
    // 2) the adjoint carries (several chunks), the reverse sweep and the reductions
    BwdArgs a;
    a.B = batch; a.L = seqlen; a.D = dim;
    a.x = x; a.delta = delta; a.z = z; a.dy = dy; a.Bm = B; a.Cm = C;
    a.A = A; a.Dskip = Dskip; a.h0 = h0; a.dh_last = dh_last;
    a.dx = dx; a.ddelta = ddelta; a.dz = dz; a.dB = dB; a.dC = dC;
    a.dA = dA; a.dD = Dskip ? dD : nullptr; a.dh0 = dh0;
    a.softplus = delta_softplus;
    a.nblk = p.nblk;
    a.n_chunks = p.n_chunks;
    a.chunk_len = p.chunk_len;
    a.ckpt = checkpoints ? const_cast<float *>(checkpoints) : reinterpret_cast<float *>(ws + p.ckpt_off);
    a.partBC = reinterpret_cast<float *>(ws + p.partBC_off);
    a.partA = reinterpret_cast<float *>(ws + p.partA_off);
    a.partD = reinterpret_cast<float *>(ws + p.partD_off);
    a.dbias = delta_bias;
    a.ddbias = delta_bias ? ddelta_bias : nullptr;
    a.partDB = reinterpret_cast<float *>(ws + p.partDB_off);
    a.lc_P = p.n_chunks > 1 ? reinterpret_cast<float *>(ws + p.lcP_off) : nullptr;
    a.lc_H = p.n_chunks > 1 ? reinterpret_cast<float *>(ws + p.lcH_off) : nullptr;
    e = launch_scan_bwd(a, discretization, bf16, z != nullptr, s);
    return e == hipSuccess ? SSM_OK : hip_fail("scan backward launch", e);
}

extern "C" int ssm_conv1d_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t width, int dtype,
                              const void *x, const float *w, const float *bias, const void *state_in,
                              void *y, void *state_out, int silu, void *stream) {
    using namespace ssm;
    clear_error();
    int st = check_conv1d_fwd(batch, seqlen, dim, width, dtype, x, w, bias, state_in, y, state_out, silu);
    if (st != SSM_OK) return st;
    if (batch == 0 || dim == 0 || (seqlen == 0 && (!state_out || width == 1))) return SSM_OK;
    ConvArgs a;
    a.B = batch; a.L = seqlen; a.D = dim; a.W = static_cast<int>(width);
    a.x = x; a.w = w; a.bias = bias; a.state_in = state_in; a.y = y; a.state_out = state_out; a.silu = silu;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // (with seqlen == 0 only the state passes through)
    hipError_t e = launch_conv1d_fwd(a, dtype == SSM_DTYPE_BF16, s);
    return e == hipSuccess ? SSM_OK : hip_fail("conv1d launch", e);
}

extern "C" size_t ssm_conv1d_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t width,
                                                 int dtype) {
    (void)dtype;
    return ssm::conv1d_bwd_ws_bytes(batch, seqlen, dim, width);
}

extern "C" int ssm_conv1d_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t width, int dtype,
                              const void *x, const float *w, const float *bias, const void *state_in,
                              const void *dy, void *dx, float *dw, float *dbias, void *dstate, int silu,
                              void *workspace, size_t workspace_bytes, void *stream) {
    using namespace ssm;
    clear_error();
    int st = check_conv1d_bwd(batch, seqlen, dim, width, dtype, x, w, bias, state_in, dy, dx, dw, dbias, dstate,
                              silu, workspace, workspace_bytes);
    if (st != SSM_OK) return st;
    if (batch == 0 || dim == 0) return SSM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (width == 1) dstate = nullptr;
    hipError_t e;
    if (seqlen == 0) {
        // no steps: every gradient is zero
        auto zero = [&](void *p, int64_t bytes) {
            if (!p || bytes <= 0) return hipSuccess;
            const int64_t n = bytes / 2;
            hipLaunchKernelGGL(zero16_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                               static_cast<uint16_t *>(p), n);
            return hipGetLastError();
        };
        e = zero(dw, dim * width * 4);
        if (e == hipSuccess) e = zero(dbias, dim * 4);
        if (e == hipSuccess) e = zero(dstate, batch * dim * (width - 1) * static_cast<int64_t>(dtype_size(dtype)));
        return e == hipSuccess ? SSM_OK : hip_fail("zero fill launch", e);
    }
    ConvArgs a;
    a.B = batch; a.L = seqlen; a.D = dim; a.W = static_cast<int>(width);
    a.x = x; a.w = w; a.bias = bias; a.state_in = state_in; a.y = nullptr; a.state_out = nullptr; a.silu = silu;
    a.dy = dy; a.dx = dx; a.dw = dw; a.dbias = dbias; a.dstate = dstate;
    a.part = static_cast<float *>(workspace);
    e = launch_conv1d_bwd(a, dtype == SSM_DTYPE_BF16, s);
    return e == hipSuccess ? SSM_OK : hip_fail("conv1d backward launch", e);
}

extern "C" int ssm_conv1d_update(int64_t batch, int64_t dim, int64_t width, int dtype, void *state,
                                 const void *x, const float *w, const float *bias, void *y, int silu,
                                 void *stream) {
    using namespace ssm;
    clear_error();
    int st = check_conv1d_update(batch, dim, width, dtype, state, x, w, bias, y, silu);
    if (st != SSM_OK) return st;
    if (batch == 0 || dim == 0) return SSM_OK;
    ConvArgs a;
    a.B = batch; a.L = 1; a.D = dim; a.W = static_cast<int>(width);
    a.x = x; a.w = w; a.bias = bias; a.state_in = nullptr; a.y = y; a.state_out = state; a.silu = silu;
    hipError_t e = launch_conv1d_update(a, dtype == SSM_DTYPE_BF16, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SSM_OK : hip_fail("conv1d update launch", e);
}

extern "C" int ssm_ssd_fwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                           int dtype, const void *x, const void *delta, const float *A, const void *B,
                           const void *C, const float *Dskip, const void *z, const float *delta_bias,
                           const float *h0, float *h_last, void *y, int delta_softplus, void *stream) {
    using namespace ssm;
    clear_error();
    int st = check_ssd(batch, seqlen, nheads, headdim, dstate, dtype, x, delta, A, B, C, Dskip, z, delta_bias,
                       h0, h_last, y, delta_softplus);
    if (st != SSM_OK) return st;
    if (batch == 0 || nheads == 0) return SSM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (seqlen == 0) {
        if (!h_last) return SSM_OK;
        const int64_t n = batch * nheads * headdim * dstate;
        hipLaunchKernelGGL(fill_state_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                           h_last, h0, n);
        hipError_t e = hipGetLastError();
        return e == hipSuccess ? SSM_OK : hip_fail("fill_state launch", e);
    }
    SsdArgs a;
    a.B = batch; a.L = seqlen; a.H = nheads;
    a.x = x; a.delta = delta; a.z = z; a.Bm = B; a.Cm = C;
    a.A = A; a.Dskip = Dskip; a.dbias = delta_bias; a.h0 = h0; a.h_last = h_last; a.y = y;
    a.softplus = delta_softplus;
    hipError_t e = launch_ssd(a, s);
    return e == hipSuccess ? SSM_OK : hip_fail("ssd launch", e);
}
