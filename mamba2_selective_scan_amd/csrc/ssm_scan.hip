// ssm_scan.hip -- the C ABI (include/ssm_scan.h) over the gfx950 scan kernel.
//
// Host side only: validate sizes and pointers, pick the compiled kernel shape
// for the state size, and enqueue one launch on the caller's stream.  Nothing
// here allocates device memory or synchronizes.
#include "ssm_scan.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <vector>

#include "correct_mfma.hpp"
#include "decode_kernel.hpp"
#include "scan_kernel.hpp"
#include "ssd_kernel.hpp"
#include "status.hpp"

namespace ssm {

thread_local hipError_t t_last_hip_error = hipSuccess;

int hip_fail(hipError_t err, int code) {
    t_last_hip_error = err;
    return code;
}

}  // namespace ssm

namespace {

using ssm::hip_fail;
using ssm::t_last_hip_error;

using ssm::kThreads;
using ssm::ScanArgs;
using ssm::Mode;
using ssm::Shape;

// One row of the shape table: state sizes up to n_max use R lanes per row,
// J float4 groups per lane and CT tokens per chunk for prefill, and DR lanes
// with DJ groups per lane for decode.  R lanes hold 4*R*J >= N elements.
// Prefill keeps E = 4J at 4..16 registers and the double-buffered staging
// under ~80 KB of the 160 KB LDS.  Decode is one pass over the state, so it
// favours more float4 loads in flight per lane (measured on MI355X at
// N = 128: 8 lanes x 16 elements beat 16 x 8 by 3%, 32 x 4 and 4 x 32 lost
// 12-17%).  The two halves of a time-split prefill run with half the chunk
// (SCT = CT / 2), so four workgroups fit in one CU's LDS.
struct ShapeRow {
    int n_max, R, J, CT, DR, DJ;
};
constexpr ShapeRow kShapes[] = {
    {16, 4, 1, 32, 4, 1},
    {32, 8, 1, 32, 8, 1},
    {64, 16, 1, 32, 16, 1},
    {128, 16, 2, 32, 8, 4},
    {256, 16, 4, 16, 16, 4},
    {512, 32, 4, 8, 32, 4},
    {1024, 64, 4, 4, 64, 4},
};
static_assert(kShapes[sizeof(kShapes) / sizeof(kShapes[0]) - 1].n_max == SSM_SCAN_MAX_D_STATE,
              "the table must cover every supported state size");

const ShapeRow *shape_for(int N) {
    for (const ShapeRow &row : kShapes)
        if (N <= row.n_max) return &row;
    return nullptr;
}

constexpr int kMaxDevices = 64;

// Opt kernel K in to more than 64 KB of dynamic LDS, once per device (the tag
// type gives every kernel its own flags).
template <class K>
int opt_in_lds(const void *kern, int lds_bytes) {
    if (lds_bytes <= 64 * 1024) return SSM_OK;
    static std::atomic<uint8_t> opted[kMaxDevices];
    int dev = 0;
    const hipError_t derr = hipGetDevice(&dev);
    if (derr != hipSuccess) return hip_fail(derr, SSM_ERR_LAUNCH);
    if (dev < 0 || dev >= kMaxDevices) return SSM_ERR_UNSUPPORTED;
    if (!opted[dev].load(std::memory_order_acquire)) {
        const hipError_t aerr = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
        if (aerr != hipSuccess) return hip_fail(aerr, SSM_ERR_LAUNCH);
        opted[dev].store(1, std::memory_order_release);
    }
    return SSM_OK;
}

template <class S, bool VEC, Mode MODE, int OPT> struct ScanKernelTag {};

}  // namespace

// Scratch of ssm_scan_prefill_static: one copy on each GPU, for the life of
// the process.  In host code its name is only a handle; kernels get the
// device address that static_scratch() looks up.
static __device__ __align__(256) char scratch[SSM_SCAN_STATIC_SCRATCH_BYTES];

namespace {

std::atomic<char *> g_scratch_addr[kMaxDevices];

// The current GPU's copy of `scratch`, looked up on the first call there.
int static_scratch(char **out) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return hip_fail(err, SSM_ERR_LAUNCH);
    if (dev < 0 || dev >= kMaxDevices) return SSM_ERR_UNSUPPORTED;
    char *p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        void *addr = nullptr;
        err = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return hip_fail(err, SSM_ERR_LAUNCH);
        if (!addr || reinterpret_cast<uintptr_t>(addr) % 256 != 0) return SSM_ERR_LAUNCH;
        p = static_cast<char *>(addr);
        g_scratch_addr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return SSM_OK;
}

template <class S, bool VEC, Mode MODE, int OPT = 0>
int launch(const ScanArgs &a, hipStream_t stream) {
    const void *kern = reinterpret_cast<const void *>(&ssm::scan_kernel<S, VEC, MODE, OPT>);
    const int lds_bytes = S::lds_floats(MODE, VEC) * int(sizeof(float));
    const int orc = opt_in_lds<ScanKernelTag<S, VEC, MODE, OPT>>(kern, lds_bytes);
    if (orc != SSM_OK) return orc;
    ScanArgs args = a;
    void *params[] = {&args};
    const hipError_t err = hipLaunchKernel(kern, dim3(unsigned(a.n_blocks)), dim3(kThreads), params,
                                           size_t(lds_bytes), stream);
    return err == hipSuccess ? SSM_OK : hip_fail(err, SSM_ERR_LAUNCH);
}

// The decode step on the vector path with no option bits (decode_kernel.hpp).
template <class S>
int launch_decode(const ScanArgs &a, hipStream_t stream) {
    ScanArgs args = a;
    void *params[] = {&args};
    const hipError_t err = hipLaunchKernel(reinterpret_cast<const void *>(&ssm::decode_kernel<S>),
                                           dim3(unsigned(a.n_blocks)), dim3(kThreads), params, 0, stream);
    return err == hipSuccess ? SSM_OK : hip_fail(err, SSM_ERR_LAUNCH);
}

// Calls f.template run<R, J, CT, DR, DJ>() for the table row: the compile-time
// shapes are read from kShapes itself, so the kernels and the host geometry
// (geo_for) cannot disagree.
template <int IDX, class F>
int run_row(F &&f) {
    constexpr ShapeRow r = kShapes[IDX];
    return f.template run<r.R, r.J, r.CT, r.DR, r.DJ>();
}
template <class F>
int with_row(const ShapeRow &row, F &&f) {
    constexpr int n_rows = int(sizeof(kShapes) / sizeof(kShapes[0]));
    static_assert(n_rows == 7, "one case per table row below");
    const int idx = int(&row - kShapes);
    switch (idx) {
    case 0: return run_row<0>(f);
    case 1: return run_row<1>(f);
    case 2: return run_row<2>(f);
    case 3: return run_row<3>(f);
    case 4: return run_row<4>(f);
    case 5: return run_row<5>(f);
    case 6: return run_row<6>(f);
    default: return SSM_ERR_UNSUPPORTED;
    }
}

// What a launch computes: a whole-sequence prefill (with the table's chunk, or
// half of it), a decode step, or one of the two kernel halves of a time-split
// prefill (segment scans, corrections).
enum class Kind { kPrefill, kPrefillHalf, kDecode, kSegScan, kCorrect };

constexpr int seg_chunk(int CT) { return CT / 2 > 2 ? CT / 2 : 2; }

// Whole-sequence prefill or decode with option bits OPT (A per state element,
// snapshots), vector or scalar path.
template <class S, Mode MODE>
int launch_opt(const ScanArgs &a, bool vec, int opt, hipStream_t stream) {
    switch (opt) {
    case 0: return vec ? launch<S, true, MODE, 0>(a, stream) : launch<S, false, MODE, 0>(a, stream);
    case 1: return vec ? launch<S, true, MODE, 1>(a, stream) : launch<S, false, MODE, 1>(a, stream);
    case 2: return vec ? launch<S, true, MODE, 2>(a, stream) : launch<S, false, MODE, 2>(a, stream);
    case 3: return vec ? launch<S, true, MODE, 3>(a, stream) : launch<S, false, MODE, 3>(a, stream);
    default: return SSM_ERR_UNSUPPORTED;
    }
}

struct Launch {
    const ScanArgs &a;
    bool vec;
    Kind kind;
    hipStream_t stream;
    int opt;
    template <int R, int J, int CT, int DR, int DJ>
    int run() const {
        constexpr int SCT = seg_chunk(CT);
        switch (kind) {
        case Kind::kDecode:
            if (vec && opt == 0) return launch_decode<Shape<DR, DJ, 1>>(a, stream);
            return launch_opt<Shape<DR, DJ, 1>, Mode::kDecode>(a, vec, opt, stream);
        case Kind::kPrefill: return launch_opt<Shape<R, J, CT>, Mode::kPrefill>(a, vec, opt, stream);
        case Kind::kPrefillHalf:
            return vec ? launch<Shape<R, J, SCT>, true, Mode::kPrefill>(a, stream)
                       : launch<Shape<R, J, SCT>, false, Mode::kPrefill>(a, stream);
        case Kind::kSegScan:
            return vec ? launch<Shape<R, J, SCT>, true, Mode::kSegScan>(a, stream)
                       : launch<Shape<R, J, SCT>, false, Mode::kSegScan>(a, stream);
        case Kind::kCorrect:
            return vec ? launch<Shape<R, J, SCT>, true, Mode::kCorrect>(a, stream)
                       : launch<Shape<R, J, SCT>, false, Mode::kCorrect>(a, stream);
        }
        return SSM_ERR_UNSUPPORTED;
    }
};

struct LdsBytes {
    bool vec;
    Kind kind;
    template <int R, int J, int CT, int DR, int DJ>
    int run() const {
        constexpr int SCT = seg_chunk(CT);
        int floats = 0;
        switch (kind) {
        case Kind::kDecode: floats = Shape<DR, DJ, 1>::lds_floats(Mode::kDecode, vec); break;
        case Kind::kPrefill: floats = Shape<R, J, CT>::lds_floats(Mode::kPrefill, vec); break;
        case Kind::kPrefillHalf: floats = Shape<R, J, SCT>::lds_floats(Mode::kPrefill, vec); break;
        case Kind::kSegScan: floats = Shape<R, J, SCT>::lds_floats(Mode::kSegScan, vec); break;
        case Kind::kCorrect: floats = Shape<R, J, SCT>::lds_floats(Mode::kCorrect, vec); break;
        }
        return int(sizeof(float)) * floats;
    }
};

// Lanes per row, elements per lane, rows per workgroup and chunk of a launch.
struct Geo {
    int R, E, RB, CT;
};
Geo geo_for(const ShapeRow &row, Kind kind) {
    const bool decode = kind == Kind::kDecode;
    const int R = decode ? row.DR : row.R;
    const int J = decode ? row.DJ : row.J;
    // half-chunk prefills and segment scans take seg_chunk(CT)
    const int CT = decode ? 1 : (kind == Kind::kPrefill ? row.CT : seg_chunk(row.CT));
    return Geo{R, 4 * J, ssm::kWaves * (64 / R), CT};
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The vector (float4) path: whole float4 groups of a state row and of a row
// block, and one chunk's B, C, x and dt within the 32-bit byte range of the
// buffer descriptors that stage them (chunks of at most 32 tokens).
bool vec_dims(const ssm_scan_dims *d) {
    constexpr int64_t kChunkBytes = 32 * int64_t(sizeof(float));
    return d->d_state % 4 == 0 && d->head_dim % 4 == 0 &&
           int64_t(d->n_heads) * d->head_dim * kChunkBytes < INT32_MAX &&
           int64_t(d->n_groups) * d->d_state * kChunkBytes < INT32_MAX;
}

int check_dims(const ssm_scan_dims *d) {
    if (!d) return SSM_ERR_NULL;
    if (d->n_heads <= 0 || d->head_dim <= 0 || d->d_state <= 0 || d->n_groups <= 0)
        return SSM_ERR_DIMS;
    if (d->n_heads % d->n_groups != 0) return SSM_ERR_DIMS;
    if (d->d_state > SSM_SCAN_MAX_D_STATE) return SSM_ERR_UNSUPPORTED;
    return SSM_OK;
}

// Whole-sequence prefill: the table's chunk, unless the grid would not fit on
// the GPU at once with it but would with half the chunk (half the LDS per
// workgroup).  A grid that runs in two rounds makes its last workgroups --
// often a batch's longest sequences, at the end of the grid -- wait for the
// first round, so their token chains run back to back (measured on the mixed
// batch, 8 sequences up to 150 tokens at H 16, P 96, N 100: 768 workgroups,
// 512 resident at 74 KB of LDS each).  Counted from LDS alone (at most four
// workgroups of four wavefronts per CU; every gfx950 part has 256 CUs), so
// the choice needs no device query.
constexpr int64_t kCus = 256;
constexpr int kLdsPerCu = 160 * 1024;
int64_t resident_per_cu(int lds_bytes) {
    const int64_t by_lds = lds_bytes > 0 ? kLdsPerCu / lds_bytes : 4;
    return std::min<int64_t>(4, by_lds);
}
Kind prefill_kind(const ShapeRow &row, bool vec, int opt, int64_t n_blocks) {
    if (opt != 0) return Kind::kPrefill;
    const int lds_full = with_row(row, LdsBytes{vec, Kind::kPrefill});
    const int lds_half = with_row(row, LdsBytes{vec, Kind::kPrefillHalf});
    const bool two_rounds = n_blocks > kCus * resident_per_cu(lds_full);
    const bool one_round_half = n_blocks <= kCus * resident_per_cu(lds_half);
    return two_rounds && one_round_half ? Kind::kPrefillHalf : Kind::kPrefill;
}

// How a prefill is cut over time.  A single long sequence exposes only
// H * P rows, one wavefront per SIMD at the headline geometry; cutting it into
// n_segs segments multiplies the wavefronts by n_segs.  Auto mode, for the
// register segment scan: cut when the whole-sequence launch would give fewer
// than 2 wavefronts per SIMD (1024 SIMDs), aiming at 4; for the matrix-core
// segment scan (shapes it covers): aim at 2 wavefronts per SIMD of its own
// geometry (4 waves per 64 rows of a head).  Segments have at least 256 tokens
// in the register form, 128 in the matrix-core form.
struct SegPlan {
    int n_segs, seg_len;
};
constexpr int64_t kTargetWaves = 4096;
constexpr int64_t kSsdTargetWaves = 2048;  // matrix-core segment scans
constexpr int kMinSegTokens = 256;
// the matrix-core split costs three launches and a state pass per segment: on
// the headline geometry one pass still wins below about 256 tokens (1 x 200:
// 27.5 us in one pass, 36-47 us split) and 128-token segments win above it
// (1 x 512: 53 us in 4 segments against 62 in one pass)
constexpr int kSsdMinSegTokens = 128;
constexpr int kSsdStateGroup = 16;         // tokens per operand group of the state pass (4 waves/SIMD)
constexpr int kSsdStateSplit128 = 1;       // N = 128: workgroups per state-column range

// The chunked matrix-core segment scan covers N <= 128 with whole 16-row
// tiles, on the vector path (16-byte aligned arrays, N % 4 == 0).  The state
// columns are padded with zeros to whole 16-column tiles inside the kernels
// (N = 100 runs as 7 tiles in the scan pass, 8 in the state pass); memory
// holds only the N real ones.
bool ssd_shape(const ssm_scan_dims *d) {
    const int N = d->d_state;
    // a window of tokens' x and B must fit 32-bit buffer offsets
    const int64_t span = int64_t(ssm::kSsdWindow + 64) * int64_t(sizeof(float));
    return N % 4 == 0 && N <= 128 && d->head_dim % 16 == 0 &&
           int64_t(d->n_heads) * d->head_dim * span < INT32_MAX &&
           int64_t(d->n_groups) * N * span < INT32_MAX;
}
bool ssd_eligible(const ssm_scan_dims *d, bool vec) { return vec && ssd_shape(d); }
// The scan pass takes two 16-row tiles per wave (128-row windows) when a
// wave's 32 rows stay in one head, else one (64-row windows).
int ssd_tiles(const ssm_scan_dims *d) { return d->head_dim % 32 == 0 ? 2 : 1; }
// Scan-pass windows per B/C group (the last one may be cut short).
int64_t ssd_windows(const ssm_scan_dims *d) {
    const int64_t group_rows = int64_t(d->n_heads / d->n_groups) * d->head_dim;
    const int64_t rbw = 64 * ssd_tiles(d);
    return (group_rows + rbw - 1) / rbw;
}
// Scan-pass kernel, its LDS floats and its LDS opt-in for state tiles NT and
// tiles per wave TW.
using OptIn = int (*)(const void *, int);
template <int NT, int TW> struct SsdScanTag {};
template <int NT, int TW>
void ssd_scan_pick(const void **kern, int *lds, OptIn *opt_in = nullptr) {
    *kern = reinterpret_cast<const void *>(&ssm::ssd_scan_kernel<NT, TW>);
    *lds = ssm::SsdScanShape<NT, TW>::lds_floats();
    if (opt_in) *opt_in = &opt_in_lds<SsdScanTag<NT, TW>>;
}
// 16-column state tiles of the scan pass (N rounded up).
int ssd_scan_tiles(const ssm_scan_dims *d) { return (d->d_state + 15) / 16; }
template <int TW>
void ssd_scan_tw(int nt, const void **kern, int *lds, OptIn *opt_in) {
    switch (nt) {
    case 1: ssd_scan_pick<1, TW>(kern, lds, opt_in); break;
    case 2: ssd_scan_pick<2, TW>(kern, lds, opt_in); break;
    case 3: ssd_scan_pick<3, TW>(kern, lds, opt_in); break;
    case 4: ssd_scan_pick<4, TW>(kern, lds, opt_in); break;
    case 5: ssd_scan_pick<5, TW>(kern, lds, opt_in); break;
    case 6: ssd_scan_pick<6, TW>(kern, lds, opt_in); break;
    case 7: ssd_scan_pick<7, TW>(kern, lds, opt_in); break;
    default: ssd_scan_pick<8, TW>(kern, lds, opt_in); break;
    }
}
void ssd_scan_for(const ssm_scan_dims *d, const void **kern, int *lds, OptIn *opt_in = nullptr) {
    if (ssd_tiles(d) == 2) ssd_scan_tw<2>(ssd_scan_tiles(d), kern, lds, opt_in);
    else ssd_scan_tw<1>(ssd_scan_tiles(d), kern, lds, opt_in);
}

SegPlan plan_segments(const ssm_scan_dims *d, const ShapeRow &row, int32_t n_seqs,
                      int32_t max_seqlen, int32_t requested) {
    const int sct = seg_chunk(row.CT);
    if (requested == 1 || max_seqlen <= sct || n_seqs <= 0) return SegPlan{1, 0};
    int64_t K;
    if (requested > 1) {
        K = requested;
    } else if (ssd_shape(d)) {
        // matrix-core segments: a scan-pass workgroup of four waves per window
        // of a group's rows; aim at two waves per SIMD (measured at 1 x 4096,
        // H64 P64 N128, two tiles per wave: 16 segments 0.169 ms, 12: 0.194,
        // 8: 0.176)
        const int64_t waves = int64_t(n_seqs) * ssm::kWaves * d->n_groups * ssd_windows(d);
        if (waves >= kSsdTargetWaves) return SegPlan{1, 0};
        K = (kSsdTargetWaves + waves - 1) / waves;
        K = std::min<int64_t>(K, max_seqlen / kSsdMinSegTokens);
    } else {
        const int RB = ssm::kWaves * (64 / row.R);
        const int64_t waves = int64_t(n_seqs) * d->n_heads * ((d->head_dim + RB - 1) / RB) * ssm::kWaves;
        if (2 * waves >= kTargetWaves) return SegPlan{1, 0};
        K = (kTargetWaves + waves - 1) / waves;
        K = std::min<int64_t>(K, max_seqlen / kMinSegTokens);
    }
    K = std::min<int64_t>(K, (int64_t(max_seqlen) + sct - 1) / sct);
    if (K < 2) return SegPlan{1, 0};
    const int64_t per = (max_seqlen + K - 1) / K;
    // whole chunks per segment, unless rounding up would lose a segment
    int seg_len = int((per + sct - 1) / sct * sct);
    if ((int64_t(max_seqlen) + seg_len - 1) / seg_len < K) seg_len = int(per);
    const int n_segs = int((int64_t(max_seqlen) + seg_len - 1) / seg_len);
    return n_segs < 2 ? SegPlan{1, 0} : SegPlan{n_segs, seg_len};
}

// Workspace carve-up for a split prefill: 256-byte aligned pieces.
struct WsLayout {
    size_t state, dtot, dcum, total;
};
size_t round256(size_t v) { return (v + 255) / 256 * 256; }
WsLayout ws_layout(const ssm_scan_dims *d, int32_t n_seqs, int32_t n_tokens, int n_segs) {
    WsLayout w{};
    const size_t seg_entries = size_t(n_seqs) * size_t(n_segs) * size_t(d->n_heads);
    w.state = 0;
    w.dtot = round256(seg_entries * size_t(d->head_dim) * size_t(d->d_state) * sizeof(float));
    w.dcum = w.dtot + round256(seg_entries * sizeof(float));
    w.total = w.dcum + round256(size_t(n_tokens) * size_t(d->n_heads) * sizeof(float)) + 256;
    return w;
}

// Shared body of every scan once the arguments are known valid.  With
// plan.n_segs > 1, `ws` (256-byte aligned, ws_layout() bytes) receives the
// segment end states and their total (and, for the register path, running)
// decays, and three kernels run: on the matrix-core path the segment state
// pass, the combine pass and the segment scans from the carried-in states;
// otherwise the segment scans, the combine pass and the corrections.
int scan_common(const ssm_scan_dims *d, const ssm_scan_options *opts, int32_t n_seqs,
                int32_t n_tokens, const int32_t *cu_seqlens, const int32_t *slot,
                const uint8_t *fresh, const float *x, const float *dt, const float *A,
                const float *B, const float *C, float *state, float *y, bool decode,
                SegPlan plan, char *ws, void *stream_ptr) {
    const ssm_scan_options none{};
    if (!opts) opts = &none;
    const int opt = (opts->a_per_state ? ssm::OPT_A_PER_STATE : 0) |
                    (opts->snapshots ? ssm::OPT_SNAPSHOTS : 0);
    if (opt) plan = SegPlan{1, 0};           // these options run whole sequences
    const ShapeRow *row = shape_for(d->d_state);
    if (!row) return SSM_ERR_UNSUPPORTED;
    const bool split = !decode && plan.n_segs > 1;
    Kind kind = decode ? Kind::kDecode : (split ? Kind::kSegScan : Kind::kPrefill);
    const int RB = geo_for(*row, kind).RB;       // the same for every prefill chunk
    const int64_t n_row_blocks = (int64_t(d->head_dim) + RB - 1) / RB;
    const int64_t n_blocks = int64_t(n_seqs) * (split ? plan.n_segs : 1) * d->n_heads * n_row_blocks;
    if (n_blocks > INT32_MAX) return SSM_ERR_UNSUPPORTED;

    const void *fptrs[] = {x, dt, A, B, C, state, y, opts->dt_bias, opts->snapshots};
    bool vec = vec_dims(d);
    for (const void *p : fptrs) {
        if (p && !aligned(p, 4)) return SSM_ERR_ALIGN;
        if (p && !aligned(p, 16)) vec = false;
    }
    if (!aligned(slot, 4) || (cu_seqlens && !aligned(cu_seqlens, 4))) return SSM_ERR_ALIGN;
    if (kind == Kind::kPrefill) kind = prefill_kind(*row, vec, opt, n_blocks);

    ScanArgs a{};
    a.cu_seqlens = cu_seqlens;
    a.slot = slot;
    a.fresh = fresh;
    a.x = x;
    a.dt = dt;
    a.A = A;
    a.B = B;
    a.C = C;
    a.state = state;
    a.y = y;
    a.H = d->n_heads;
    a.P = d->head_dim;
    a.N = d->d_state;
    a.G = d->n_groups;
    a.heads_per_group = d->n_heads / d->n_groups;
    a.n_row_blocks = int32_t(n_row_blocks);
    a.n_blocks = int32_t(n_blocks);
    a.n_segs = split ? plan.n_segs : 1;
    a.seg_len = split ? plan.seg_len : 0;
    a.dt_bias = opts->dt_bias;
    a.dt_softplus = opts->dt_softplus ? 1 : 0;
    a.snapshots = opts->snapshots;
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    if (!split) return with_row(*row, Launch{a, vec, kind, stream, opt});

    const WsLayout w = ws_layout(d, n_seqs, n_tokens, plan.n_segs);
    a.ws_state = reinterpret_cast<float *>(ws + w.state);
    a.ws_dtot = reinterpret_cast<float *>(ws + w.dtot);
    a.ws_dcum = reinterpret_cast<float *>(ws + w.dcum);
    auto combine = [&](int into_slot) -> int {
        const int64_t units = int64_t(n_seqs) * d->n_heads * d->head_dim * d->d_state / (vec ? 4 : 1);
        const int64_t grid = (units + kThreads - 1) / kThreads;
        if (grid > INT32_MAX) return SSM_ERR_UNSUPPORTED;
        const void *kern = vec ? reinterpret_cast<const void *>(&ssm::combine_kernel<true>)
                               : reinterpret_cast<const void *>(&ssm::combine_kernel<false>);
        ScanArgs args = a;
        int64_t n_units = units;
        int slot_flag = into_slot;
        void *params[] = {&args, &n_units, &slot_flag};
        const hipError_t err =
            hipLaunchKernel(kern, dim3(unsigned(grid)), dim3(kThreads), params, 0, stream);
        return err == hipSuccess ? SSM_OK : hip_fail(err, SSM_ERR_LAUNCH);
    };
    if (ssd_eligible(d, vec)) {
        // Matrix-core path: (1) the end state of every segment but the last,
        // (2) the combine pass turns them into carried-in states, (3) every
        // segment scanned in chunked form from its carried-in state: y final,
        // the last segment's end state to the slot.
        ScanArgs sa = a;
        sa.n_row_blocks = (d->head_dim + 63) / 64;
        const int64_t per_seg = int64_t(n_seqs) * d->n_heads * sa.n_row_blocks;
        if (per_seg * plan.n_segs > INT32_MAX) return SSM_ERR_UNSUPPORTED;
        // state-pass column tiles: N rounded up to 32, 64 or 128
        const int nt = d->d_state <= 32 ? 2 : d->d_state <= 64 ? 4 : 8;
        auto pass = [&](bool states) -> int {
            const void *kern;
            int lds;
            int64_t blocks = per_seg * plan.n_segs;
            int64_t slabs = sa.n_row_blocks;     // row blocks per head, or windows per group
            if (states) {
                blocks = per_seg * (plan.n_segs - 1);
                lds = 0;                         // static LDS only
                // N = 128 splits its state columns over two workgroups
                if (nt == 8) {
                    kern = reinterpret_cast<const void *>(
                        &ssm::ssd_state_kernel<8, kSsdStateSplit128, kSsdStateGroup>);
                    blocks *= kSsdStateSplit128;
                } else if (nt == 4) {
                    kern = reinterpret_cast<const void *>(&ssm::ssd_state_kernel<4, 1, kSsdStateGroup>);
                } else {
                    kern = reinterpret_cast<const void *>(&ssm::ssd_state_kernel<2, 1, kSsdStateGroup>);
                }
            } else {
                OptIn opt_in = nullptr;
                ssd_scan_for(d, &kern, &lds, &opt_in);
                const int orc = opt_in(kern, lds * int(sizeof(float)));
                if (orc != SSM_OK) return orc;
                slabs = ssd_windows(d);
                blocks = int64_t(n_seqs) * plan.n_segs * d->n_groups * slabs;
            }
            if (blocks > INT32_MAX) return SSM_ERR_UNSUPPORTED;
            ScanArgs la = sa;
            la.n_row_blocks = int32_t(slabs);
            la.n_blocks = int32_t(blocks);
            void *params[] = {&la};
            const hipError_t err = hipLaunchKernel(kern, dim3(unsigned(blocks)), dim3(kThreads),
                                                   params, size_t(lds) * sizeof(float), stream);
            return err == hipSuccess ? SSM_OK : hip_fail(err, SSM_ERR_LAUNCH);
        };
        int rc = pass(true);
        if (rc == SSM_OK) rc = combine(0);
        if (rc == SSM_OK) rc = pass(false);
        return rc;
    }
    int rc = with_row(*row, Launch{a, vec, Kind::kSegScan, stream, 0});
    if (rc == SSM_OK) rc = combine(1);
    if (rc != SSM_OK) return rc;
    // Corrections: a dense contraction per segment, on the matrix cores when
    // the state rows split into float4 halves (N % 8 == 0, N <= 128).
    if (vec && d->d_state % 8 == 0 && d->d_state <= 128) {
        const int n_tblocks = (plan.seg_len + 127) / 128;
        // segments 1.. only: segment 0 started from the true state
        const int64_t grid = int64_t(n_seqs) * (plan.n_segs - 1) * d->n_heads * n_tblocks;
        if (grid > INT32_MAX) return SSM_ERR_UNSUPPORTED;
        const int nh = d->d_state / 2;
        const void *kern =
            nh == 16 ? reinterpret_cast<const void *>(&ssm::correct_mfma_kernel<16, true>)
          : nh < 16  ? reinterpret_cast<const void *>(&ssm::correct_mfma_kernel<16, false>)
          : nh == 32 ? reinterpret_cast<const void *>(&ssm::correct_mfma_kernel<32, true>)
          : nh < 32  ? reinterpret_cast<const void *>(&ssm::correct_mfma_kernel<32, false>)
          : nh == 64 ? reinterpret_cast<const void *>(&ssm::correct_mfma_kernel<64, true>)
                     : reinterpret_cast<const void *>(&ssm::correct_mfma_kernel<64, false>);
        ScanArgs args = a;
        int tblocks = n_tblocks;
        void *params[] = {&args, &tblocks};
        const hipError_t err =
            hipLaunchKernel(kern, dim3(unsigned(grid)), dim3(kThreads), params, 0, stream);
        return err == hipSuccess ? SSM_OK : hip_fail(err, SSM_ERR_LAUNCH);
    }
    return with_row(*row, Launch{a, vec, Kind::kCorrect, stream, 0});
}

}  // namespace

extern "C" {

int ssm_scan_prefill(const ssm_scan_dims *dims, int32_t n_seqs, int32_t n_tokens,
                     const int32_t *cu_seqlens, const int32_t *slot, const uint8_t *fresh,
                     const float *x, const float *dt, const float *A, const float *B,
                     const float *C, float *state, int32_t n_slots, float *y, void *stream) {
    const int rc = check_dims(dims);
    if (rc != SSM_OK) return rc;
    if (n_seqs < 0 || n_tokens < 0 || n_slots < 0) return SSM_ERR_DIMS;
    if (n_seqs == 0) return SSM_OK;
    if (n_slots == 0) return SSM_ERR_DIMS;
    if (!cu_seqlens || !slot || !fresh || !A || !state) return SSM_ERR_NULL;
    if (n_tokens > 0 && (!x || !dt || !B || !C || !y)) return SSM_ERR_NULL;
    return scan_common(dims, nullptr, n_seqs, n_tokens, cu_seqlens, slot, fresh, x, dt, A, B, C,
                       state, y, /*decode=*/false, SegPlan{1, 0}, nullptr, stream);
}

int ssm_scan_prefill_workspace_size(const ssm_scan_dims *dims, int32_t n_seqs, int32_t n_tokens,
                                    int32_t max_seqlen, int32_t n_segments, size_t *bytes) {
    const int rc = check_dims(dims);
    if (rc != SSM_OK) return rc;
    if (!bytes) return SSM_ERR_NULL;
    if (n_seqs < 0 || n_tokens < 0 || max_seqlen < 0 || n_segments < 0) return SSM_ERR_DIMS;
    const ShapeRow *row = shape_for(dims->d_state);
    const SegPlan plan = plan_segments(dims, *row, n_seqs, max_seqlen, n_segments);
    *bytes = plan.n_segs > 1 ? ws_layout(dims, n_seqs, n_tokens, plan.n_segs).total : 0;
    return SSM_OK;
}

int ssm_scan_prefill_opt(const ssm_scan_dims *dims, const ssm_scan_options *opts, int32_t n_seqs,
                         int32_t n_tokens, int32_t max_seqlen, int32_t n_segments,
                         const int32_t *cu_seqlens, const int32_t *slot, const uint8_t *fresh,
                         const float *x, const float *dt, const float *A, const float *B,
                         const float *C, float *state, int32_t n_slots, float *y, void *workspace,
                         size_t workspace_bytes, void *stream) {
    const int rc = check_dims(dims);
    if (rc != SSM_OK) return rc;
    if (n_seqs < 0 || n_tokens < 0 || n_slots < 0 || max_seqlen < 0 || n_segments < 0)
        return SSM_ERR_DIMS;
    if (n_seqs == 0) return SSM_OK;
    if (n_slots == 0) return SSM_ERR_DIMS;
    if (!cu_seqlens || !slot || !fresh || !A || !state) return SSM_ERR_NULL;
    if (n_tokens > 0 && (!x || !dt || !B || !C || !y)) return SSM_ERR_NULL;
    const ShapeRow *row = shape_for(dims->d_state);
    SegPlan plan = plan_segments(dims, *row, n_seqs, max_seqlen, n_segments);
    char *ws = nullptr;
    if (plan.n_segs > 1) {
        const size_t need = ws_layout(dims, n_seqs, n_tokens, plan.n_segs).total;
        if (!workspace || workspace_bytes < need) {
            plan = SegPlan{1, 0};                    // not enough room: one pass per sequence
        } else {
            const uintptr_t p = reinterpret_cast<uintptr_t>(workspace);
            ws = reinterpret_cast<char *>((p + 255) / 256 * 256);
        }
    }
    return scan_common(dims, opts, n_seqs, n_tokens, cu_seqlens, slot, fresh, x, dt, A, B, C,
                       state, y, /*decode=*/false, plan, ws, stream);
}

int ssm_scan_prefill_ws(const ssm_scan_dims *dims, int32_t n_seqs, int32_t n_tokens,
                        int32_t max_seqlen, int32_t n_segments, const int32_t *cu_seqlens,
                        const int32_t *slot, const uint8_t *fresh, const float *x,
                        const float *dt, const float *A, const float *B, const float *C,
                        float *state, int32_t n_slots, float *y, void *workspace,
                        size_t workspace_bytes, void *stream) {
    return ssm_scan_prefill_opt(dims, nullptr, n_seqs, n_tokens, max_seqlen, n_segments,
                                cu_seqlens, slot, fresh, x, dt, A, B, C, state, n_slots, y,
                                workspace, workspace_bytes, stream);
}

int ssm_scan_prefill_static(const ssm_scan_dims *dims, int32_t n_seqs, int32_t n_tokens,
                            int32_t max_seqlen, int32_t n_segments, const int32_t *cu_seqlens,
                            const int32_t *slot, const uint8_t *fresh, const float *x,
                            const float *dt, const float *A, const float *B, const float *C,
                            float *state, int32_t n_slots, float *y, void *stream) {
    const int rc = check_dims(dims);
    if (rc != SSM_OK) return rc;
    if (n_seqs < 0 || n_tokens < 0 || n_slots < 0 || max_seqlen < 0 || n_segments < 0)
        return SSM_ERR_DIMS;
    if (n_seqs == 0) return SSM_OK;
    if (n_slots == 0) return SSM_ERR_DIMS;
    if (!cu_seqlens || !slot || !fresh || !A || !state) return SSM_ERR_NULL;
    if (n_tokens > 0 && (!x || !dt || !B || !C || !y)) return SSM_ERR_NULL;
    const ShapeRow *row = shape_for(dims->d_state);
    const SegPlan plan = plan_segments(dims, *row, n_seqs, max_seqlen, n_segments);
    char *ws = nullptr;
    if (plan.n_segs > 1) {
        if (ws_layout(dims, n_seqs, n_tokens, plan.n_segs).total > SSM_SCAN_STATIC_SCRATCH_BYTES)
            return SSM_ERR_SCRATCH;
        const int src = static_scratch(&ws);
        if (src != SSM_OK) return src;
    }
    return scan_common(dims, nullptr, n_seqs, n_tokens, cu_seqlens, slot, fresh, x, dt, A, B, C,
                       state, y, /*decode=*/false, plan, ws, stream);
}

int ssm_scan_decode_opt(const ssm_scan_dims *dims, const ssm_scan_options *opts, int32_t n_seqs,
                        const int32_t *slot, const uint8_t *fresh, const float *x,
                        const float *dt, const float *A, const float *B, const float *C,
                        float *state, int32_t n_slots, float *y, void *stream) {
    const int rc = check_dims(dims);
    if (rc != SSM_OK) return rc;
    if (n_seqs < 0 || n_slots < 0) return SSM_ERR_DIMS;
    if (n_seqs == 0) return SSM_OK;
    if (n_slots == 0) return SSM_ERR_DIMS;
    if (!slot || !fresh || !A || !state || !x || !dt || !B || !C || !y) return SSM_ERR_NULL;
    return scan_common(dims, opts, n_seqs, n_seqs, nullptr, slot, fresh, x, dt, A, B, C, state,
                       y, /*decode=*/true, SegPlan{1, 0}, nullptr, stream);
}

int ssm_scan_decode(const ssm_scan_dims *dims, int32_t n_seqs, const int32_t *slot,
                    const uint8_t *fresh, const float *x, const float *dt, const float *A,
                    const float *B, const float *C, float *state, int32_t n_slots, float *y,
                    void *stream) {
    return ssm_scan_decode_opt(dims, nullptr, n_seqs, slot, fresh, x, dt, A, B, C, state, n_slots,
                               y, stream);
}

const char *ssm_scan_strerror(int code) {
    switch (code) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL: return "a required pointer is NULL";
    case SSM_ERR_DIMS: return "invalid size (non-positive dimension, negative count, or n_heads % n_groups != 0)";
    case SSM_ERR_UNSUPPORTED: return "unsupported size (d_state above the maximum, or the grid is too large)";
    case SSM_ERR_ALIGN: return "an array is not 4-byte aligned";
    case SSM_ERR_LAUNCH: return "the HIP runtime refused the kernel launch";
    case SSM_ERR_METADATA: return "invalid metadata (cu_seqlens not monotone from 0 to n_tokens, or a slot out of range or repeated)";
    case SSM_ERR_SCRATCH: return "the split needs more scratch than the library's static buffer (SSM_SCAN_STATIC_SCRATCH_BYTES) holds";
    default: return "unknown status code";
    }
}

int ssm_scan_version(void) { return SSM_SCAN_ABI_VERSION; }

int ssm_scan_last_hip_error(void) { return int(t_last_hip_error); }

const char *ssm_scan_last_hip_error_string(void) {
    return t_last_hip_error == hipSuccess ? "no error" : hipGetErrorString(t_last_hip_error);
}

int ssm_scan_check_metadata_host(int32_t n_seqs, int32_t n_tokens, const int32_t *cu_seqlens,
                                 const int32_t *slot, int32_t n_slots) {
    if (n_seqs < 0 || n_tokens < 0 || n_slots < 0) return SSM_ERR_DIMS;
    if (n_seqs == 0) return SSM_OK;
    if (!slot) return SSM_ERR_NULL;
    if (cu_seqlens) {
        if (cu_seqlens[0] != 0 || cu_seqlens[n_seqs] != n_tokens) return SSM_ERR_METADATA;
        for (int32_t s = 0; s < n_seqs; ++s)
            if (cu_seqlens[s + 1] < cu_seqlens[s]) return SSM_ERR_METADATA;
    }
    for (int32_t s = 0; s < n_seqs; ++s)
        if (slot[s] < 0 || slot[s] >= n_slots) return SSM_ERR_METADATA;
    // distinct slots: sort-free check with a bitmap over [0, n_slots)
    const int64_t words = (int64_t(n_slots) + 63) / 64;
    uint64_t small[64];
    uint64_t *seen = small;
    uint64_t *heap = nullptr;
    if (words > 64) {
        heap = new (std::nothrow) uint64_t[size_t(words)];
        if (!heap) return SSM_ERR_UNSUPPORTED;
        seen = heap;
    }
    std::memset(seen, 0, size_t(words) * sizeof(uint64_t));
    int rc = SSM_OK;
    for (int32_t s = 0; s < n_seqs && rc == SSM_OK; ++s) {
        const uint64_t bit = uint64_t(1) << (slot[s] % 64);
        uint64_t &w = seen[slot[s] / 64];
        if (w & bit) rc = SSM_ERR_METADATA;
        w |= bit;
    }
    delete[] heap;
    return rc;
}

int ssm_scan_check_metadata(int32_t n_seqs, int32_t n_tokens, const int32_t *cu_seqlens,
                            const int32_t *slot, int32_t n_slots, void *stream_ptr) {
    if (n_seqs < 0 || n_tokens < 0 || n_slots < 0) return SSM_ERR_DIMS;
    if (n_seqs == 0) return SSM_OK;
    if (!slot) return SSM_ERR_NULL;
    // Host copies (a debugging aid: this call synchronizes by design).
    std::vector<int32_t> cu_h(cu_seqlens ? size_t(n_seqs) + 1 : 0);
    std::vector<int32_t> slot_h(static_cast<size_t>(n_seqs));
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    hipError_t err = hipMemcpyAsync(slot_h.data(), slot, slot_h.size() * sizeof(int32_t),
                                    hipMemcpyDeviceToHost, stream);
    if (err == hipSuccess && cu_seqlens)
        err = hipMemcpyAsync(cu_h.data(), cu_seqlens, cu_h.size() * sizeof(int32_t),
                             hipMemcpyDeviceToHost, stream);
    if (err == hipSuccess) err = hipStreamSynchronize(stream);
    if (err != hipSuccess) return hip_fail(err, SSM_ERR_LAUNCH);
    return ssm_scan_check_metadata_host(n_seqs, n_tokens, cu_seqlens ? cu_h.data() : nullptr,
                                        slot_h.data(), n_slots);
}

int ssm_scan_query_geometry(const ssm_scan_dims *dims, int32_t n_seqs, int32_t decode,
                            int32_t aligned16, ssm_scan_geometry *out) {
    const int rc = check_dims(dims);
    if (rc != SSM_OK) return rc;
    if (!out) return SSM_ERR_NULL;
    if (n_seqs < 0) return SSM_ERR_DIMS;
    const ShapeRow *row = shape_for(dims->d_state);
    if (!row) return SSM_ERR_UNSUPPORTED;
    const bool vec = aligned16 && vec_dims(dims);
    Kind kind = decode ? Kind::kDecode : Kind::kPrefill;
    if (!decode) {
        const int64_t rb = geo_for(*row, kind).RB;
        kind = prefill_kind(*row, vec, 0, int64_t(n_seqs) * dims->n_heads * ((dims->head_dim + rb - 1) / rb));
    }
    const Geo geo = geo_for(*row, kind);
    out->lanes_per_row = geo.R;
    out->elems_per_lane = geo.E;
    out->rows_per_block = geo.RB;
    out->chunk_tokens = geo.CT;
    out->threads_per_block = kThreads;
    out->lds_bytes = with_row(*row, LdsBytes{vec, kind});
    out->blocks = int64_t(n_seqs) * dims->n_heads * ((int64_t(dims->head_dim) + geo.RB - 1) / geo.RB);
    out->vector_path = vec ? 1 : 0;
    out->segments = 1;
    out->segment_tokens = 0;
    return SSM_OK;
}

int ssm_scan_query_prefill_plan(const ssm_scan_dims *dims, int32_t n_seqs, int32_t max_seqlen,
                                int32_t n_segments, int32_t aligned16, ssm_scan_geometry *out) {
    const int rc = ssm_scan_query_geometry(dims, n_seqs, 0, aligned16, out);
    if (rc != SSM_OK) return rc;
    if (max_seqlen < 0 || n_segments < 0) return SSM_ERR_DIMS;
    const ShapeRow *row = shape_for(dims->d_state);
    const SegPlan plan = plan_segments(dims, *row, n_seqs, max_seqlen, n_segments);
    if (plan.n_segs > 1) {
        const bool vec = out->vector_path != 0;
        if (ssd_eligible(dims, vec)) {
            // matrix-core segment scan: 4 lanes hold a row's N values (l % 16 is
            // the row, l / 16 the quarter of each 16-wide state tile), 16-token
            // chunks
            out->lanes_per_row = 4;
            out->elems_per_lane = 4 * ssd_scan_tiles(dims);
            out->chunk_tokens = 16;
            // the scan pass: a window of 64 rows per tile per wave
            const void *kern;
            int lds;
            ssd_scan_for(dims, &kern, &lds);
            out->rows_per_block = 64 * ssd_tiles(dims);
            out->lds_bytes = lds * int(sizeof(float));
            out->blocks = int64_t(n_seqs) * plan.n_segs * dims->n_groups * ssd_windows(dims);
        } else {
            const Geo geo = geo_for(*row, Kind::kSegScan);
            out->chunk_tokens = geo.CT;
            out->lds_bytes = with_row(*row, LdsBytes{vec, Kind::kSegScan});
            out->blocks *= plan.n_segs;
        }
        out->segments = plan.n_segs;
        out->segment_tokens = plan.seg_len;
    }
    return SSM_OK;
}

}  // extern "C"
