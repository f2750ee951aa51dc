// Host-side argument checks and launch planning for libssm (no HIP here, so
// the same code builds with g++ under sanitizers for CPU tests).
#pragma once

#include <cstddef>
#include <cstdint>

#include "ssm.h"

namespace ssm {

constexpr int kWave = 64;            // lanes per wavefront on gfx950
constexpr int kChannelsPerBlock = 64; // one channel per lane of a wave
constexpr int kMaxWavesPerBlock = 16;
constexpr size_t kWsAlign = 256;
constexpr int64_t kCUs = 256;          // MI355X compute units
constexpr size_t kLdsPerCU = 160 * 1024;

struct ScanPlan {
    int G = 4;            // states of one channel held by one lane
    int NW = 4;           // waves per workgroup = ceil(N / G)
    int TB = 32;          // time steps staged per block
    int64_t chunk_len = 0;
    int64_t n_chunks = 1;
    size_t ws_bytes = 0;  // workspace for chunk carries (0 when n_chunks == 1)
    size_t ws_P_off = 0;  // byte offset of the per-chunk state decays [B][C-1][D][N]
    size_t ws_H_off = 0;  // byte offset of the per-chunk end states [B][C-1][D][N]
    size_t ws_BC_off = 0; // specialised kernel: byte offset of the packed fp32 B/C rows
    int64_t bc_lpad = 0;  // specialised kernel: steps per chunk in the packed B/C rows (multiple of 16)
    uint64_t blocks = 0;  // workgroups of the main scan launch
    bool fast = false;    // dstate == 16 and dim % 64 == 0: the specialised kernel runs
    size_t lds_reserve = 0;  // dynamic LDS that caps residency at one workgroup per CU
    bool structured = true;  // the Mamba kernels may take their structured-A path (device check)
    // Long chunks (chunk_len >= kLocalMinChunk): the workspace also holds what the local-scan
    // carries need (ScanArgs::ws_Hl, S_part, flags; ws_P then receives the prefix rescan's end
    // states).  run_scan uses them for the exponential discretisations.
    bool local = false;
    size_t ws_Hl_off = 0, ws_S_off = 0, ws_F_off = 0;
};
// Local-scan carries: the prefix of every chunk >= 1 that is rescanned from its carried-in
// state, and the shortest chunk for which the local-scan carries are used.
constexpr int64_t kLocalPrefix = 4096;
constexpr int64_t kLocalMinChunk = 4 * kLocalPrefix;

// Per-thread error text (ssm_last_error).
void set_error(const char *fmt, ...);
// Whether the environment variable name is set to something other than "" or "0" (read
// once per name by its callers).
bool env_flag(const char *name);
// SSM_LOG=1: one line per call on stderr describing what the entry point launches (shape,
// kernel path, plan).  Nothing is printed otherwise.
void log_call(const char *fmt, ...);
void clear_error();

// Shape and option checks + plan.  Returns an ssm_status.
int plan_scan(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
              const ssm_scan_opts *opts, ScanPlan *plan);

// Full argument check of ssm_scan_fwd (shape, pointers, alignment, overlap,
// workspace).  Returns an ssm_status; fills *plan on success.
int check_scan(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
               const void *x, const void *delta, const float *A, const void *B, const void *C,
               const float *Dskip, const void *z, const float *h0, const float *h_last,
               const void *y, int delta_softplus, const ssm_variant *variant,
               const ssm_scan_opts *opts, const void *workspace, size_t workspace_bytes,
               ScanPlan *plan);

// Full argument check of ssm_state_update.
int check_state_update(int64_t batch, int64_t dim, int64_t dstate, int dtype, const float *h,
                       const void *x, const void *delta, const float *A, const void *B,
                       const void *C, const float *Dskip, const void *z, const void *y,
                       int delta_softplus, const ssm_variant *variant);

// The discretisation of a variant (NULL = SSM_DISC_MAMBA) and its delta bias.
inline int variant_disc(const ssm_variant *v) { return v ? v->discretization : SSM_DISC_MAMBA; }
inline const float *variant_bias(const ssm_variant *v) { return v ? v->delta_bias : nullptr; }

// Workspace of ssm_scan_bwd: per-workgroup shares of dB/dC, per-(chunk, row) shares of
// dA/dD, the adjoint carries, then (last, so that a call given saved checkpoints needs
// only the part before them) the forward checkpoint pass's own workspace and the state
// checkpoints.
// Buffers of the padded backward, in workspace order: inputs, then outputs, then (with more
// than one group of 16 states) the fp32 sums of the per-channel gradients over the groups.
enum PadBuf {
    kPX, kPDelta, kPZ, kPDy, kPB, kPC, kPA, kPDskip, kPBias, kPH0, kPDhLast,
    kPDx, kPDdelta, kPDz, kPDB, kPDC, kPDA, kPDD, kPDBias, kPDh0,
    kSDx, kSDdelta, kSDz, kSDBias, kPadBufs
};

struct BwdPlan {
    int64_t nblk = 0;       // 8-step blocks of the reverse sweep
    int64_t n_chunks = 1, chunk_len = 0;   // sequence chunks (chunk_len a multiple of 16 when several)
    ScanPlan fwd;           // the checkpoint pass: the specialised forward kernel, same chunks
    size_t partBC_off = 0, partA_off = 0, partD_off = 0, partDB_off = 0;
    size_t lcP_off = 0, lcH_off = 0;   // adjoint carries (several chunks only)
    size_t fwd_off = 0;     // the forward plan's workspace (its carries and packed B/C)
    size_t ckpt_off = 0;    // checkpoints [B][nblk][16][D] fp32
    size_t ckpt_bytes = 0;
    size_t ws_bytes = 0;        // with the checkpoint pass
    size_t ws_bytes_saved = 0;  // given saved checkpoints (= fwd_off)
    // Other shapes (dstate < 16 or dim not a multiple of 64) run the same kernels on copies
    // padded to dim Dp (the next multiple of 64) and 16 states, in the workspace; the pad
    // region comes first, the native plan's workspace (of the padded shape) after it.
    bool pad = false;
    int64_t Dp = 0;
    // More than 16 states: K = ceil(dstate / 16) groups of 16, each run through the native
    // kernels on fp32 copies (the token tensors once, B, C, A and the states per group); the
    // per-channel gradients (dx, ddelta, dz, the bias's) are sums over the groups, D enters
    // in group 0 only.  K == 1 is the padded path above, on copies of the input dtype.
    int64_t K = 1;
    // K > 1 with fp32 tokens of a width that needs no padding: the tokens are read in place and
    // the per-channel gradients summed straight into the caller's outputs (no token copies)
    bool direct = false;
    size_t pad_off[kPadBufs] = {};
    size_t inner_off = 0;
};

int plan_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                  BwdPlan *plan);

// Full argument check of ssm_scan_bwd.
int check_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                   const void *x, const void *delta, const float *A, const void *B, const void *C,
                   const float *Dskip, const void *z, const float *h0, const void *dy,
                   const float *dh_last, const void *dx, const void *ddelta, const float *dA,
                   const void *dB, const void *dC, const float *dD, const void *dz, const float *dh0,
                   int delta_softplus, int discretization, const float *delta_bias,
                   const float *ddelta_bias, const float *checkpoints,
                   const void *workspace, size_t workspace_bytes, BwdPlan *plan);
// Full argument check of ssm_scan_fwd_save: ssm_scan_fwd's on the backward's chunk plan,
// plus the checkpoint output.  Fills *plan (the backward's) on success.
int check_scan_save(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                    const void *x, const void *delta, const float *A, const void *B, const void *C,
                    const float *Dskip, const void *z, const float *h0, const float *h_last,
                    const void *y, int delta_softplus, const ssm_variant *variant,
                    const float *checkpoints, const void *workspace, size_t workspace_bytes,
                    BwdPlan *plan);

// Argument checks of the convolution entry points.
int check_conv1d_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t width, int dtype,
                     const void *x, const float *w, const float *bias, const void *state_in,
                     const void *y, const void *state_out, int silu);
constexpr int kConvBwdTile = 64;   // steps per thread (and per partial sum) in the convolution's backward

// Bytes of the convolution backward's workspace (per-(row, tile) sums of dw, dbias).
size_t conv1d_bwd_ws_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t width);
int check_conv1d_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t width, int dtype,
                     const void *x, const float *w, const float *bias, const void *state_in,
                     const void *dy, const void *dx, const float *dw, const float *dbias,
                     const void *dstate, int silu, const void *workspace, size_t workspace_bytes);
int check_conv1d_update(int64_t batch, int64_t dim, int64_t width, int dtype, const void *state,
                        const void *x, const float *w, const float *bias, const void *y, int silu);

// Argument checks of the multi-head SSD scan (ssm_ssd_fwd).
int check_ssd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups, int dtype,
              const void *x, const void *delta, const float *A, const void *B, const void *C,
              const float *Dskip, const void *z, const float *delta_bias, const float *h0,
              const float *h_last, const void *y, int delta_softplus);

inline size_t dtype_size(int dtype) { return dtype == SSM_DTYPE_BF16 ? 2 : 4; }

}  // namespace ssm
