// trimul.cpp -- host side of libtrimul: argument checks, the gfx950 gate,
// weight rounding and packing, workspace carving and the three launches.
//
// Follows the fold-cp-ops README: every data-independent decision is taken at
// construction ("Use", step 2: the constructor validates and configures,
// forward makes no decisions), and a device of the wrong architecture is
// refused up front with a message naming what was found ("Hardware" section)
// rather than failing later inside a launch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "trimul.h"
#include "trimul_internal.h"
#include "trimul_launch.hpp"
#include "trimul_plans.hpp"

struct trimul_handle {
    trimul::Params p;
    void* dev_mem;
    int device;
    std::string arch;                   // device architecture name (cache key)
    std::mutex mu;                      // guards plans
    std::vector<trimul::PlanEntry> plans;
    void* scratch;                      // this device's address of `scratch` (trimul_fwd_noalloc)
};

// Workspace of trimul_fwd_noalloc: one array per device, loaded with the
// library's code object and held until the process ends.  In host code the
// name is only a stand-in for the symbol; the device address comes from
// hipGetSymbolAddress, once per device, in trimul_create (scratch_address).
static __device__ __align__(256) unsigned char scratch[TRIMUL_NOALLOC_MAX_BYTES];

namespace {

// The last error message of this thread: a fixed buffer, so that reporting
// an error never allocates (and never throws).
thread_local char g_err[512];

trimul_status fail(trimul_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

trimul_status ok()
{
    g_err[0] = '\0';
    return TRIMUL_OK;
}

// No C++ exception crosses the C ABI: entry points whose host code allocates
// (packing, plan lists, the cache file) run through these, which turn any
// exception (in practice std::bad_alloc) into an error status.
template <typename F>
trimul_status guarded(F&& f) noexcept
{
    try {
        return f();
    } catch (...) {
        return fail(TRIMUL_ERR_INVALID_ARG, "host-side failure (out of host memory?)");
    }
}

template <typename F>
int guarded_int(F&& f, int on_error) noexcept
{
    try {
        return f();
    } catch (...) {
        fail(TRIMUL_ERR_INVALID_ARG, "host-side failure (out of host memory?)");
        return on_error;
    }
}

trimul_status hip_fail(const char* what, hipError_t e)
{
    return fail(TRIMUL_ERR_HIP, "%s failed: %s (%d)", what, hipGetErrorString(e), (int)e);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t elem_size(trimul_dtype t) { return t == TRIMUL_BF16 ? 2 : 4; }

bool width_ok(int x) { return x >= 32 && x <= 256 && x % 32 == 0; }

// Round to nearest even, as the hardware conversion does.
uint16_t f32_to_bf16(float f)
{
    uint32_t u;
    std::memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

float bf16_to_f32(uint16_t h)
{
    const uint32_t u = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// Folded output GEMM for the bf16 kernels that apply LayerNorm algebraically:
// rows d of W (rows x K, fp32) become bf16(W[d][k] * gamma[k]), and each row
// gets the correction terms S_d = sum_k of the folded bf16 row and
// T_d = sum_k W[d][k] * beta[k], each split as high = bf16(v), low = bf16(v - high).
void fold_rows(const float* W, const float* gamma, const float* beta, int rows, int K,
               uint16_t* wf, uint16_t* x)
{
    for (int d = 0; d < rows; ++d) {
        double S = 0.0, T = 0.0;
        for (int k = 0; k < K; ++k) {
            const uint16_t h = f32_to_bf16((float)((double)W[(size_t)d * K + k] * gamma[k]));
            wf[(size_t)d * K + k] = h;
            S += bf16_to_f32(h);
            T += (double)W[(size_t)d * K + k] * beta[k];
        }
        const uint16_t sh = f32_to_bf16((float)S), th = f32_to_bf16((float)T);
        const uint16_t sl = f32_to_bf16((float)(S - bf16_to_f32(sh)));
        const uint16_t tl = f32_to_bf16((float)(T - bf16_to_f32(th)));
        const uint16_t row[8] = {sh, sl, sh, th, tl, th, 0, 0};
        std::memcpy(x + (size_t)d * 8, row, sizeof row);
    }
}

// Folded projection for the bf16 projection kernel, rows in the kernel's order
// (stages of 16 p rows then the same channels' 16 g rows).  Row r becomes
// bf16(s W[r][k] gamma[k]) and gets the fp32 vector (T, T, T, T) with
// T = s sum_k W[r][k] beta[k], where s = -log2(e) for gate rows and 1 for the
// others: the kernel starts each accumulator at T, so a p accumulator ends at
// p and a g accumulator at -log2(e) g, the exponent of the sigmoid's 2^x form.
void fold_projection_rows(const float* W, const float* gamma, const float* beta, int rows, int K,
                          uint16_t* wf, float* tv)
{
    const double log2e = 1.4426950408889634;
    for (int r = 0; r < rows; ++r) {
        const double sgn = (r % 32) >= 16 ? -log2e : 1.0;
        double T = 0.0;
        for (int k = 0; k < K; ++k) {
            const double w = W[(size_t)r * K + k];
            wf[(size_t)r * K + k] = f32_to_bf16((float)(sgn * w * gamma[k]));
            T += w * beta[k];
        }
        for (int i = 0; i < 4; ++i) tv[(size_t)r * 4 + i] = (float)(sgn * T);
    }
}

void put(std::vector<uint8_t>& dst, size_t off_elems, float v, trimul_dtype t)
{
    if (t == TRIMUL_BF16) {
        uint16_t h = f32_to_bf16(v);
        std::memcpy(dst.data() + off_elems * 2, &h, 2);
    } else {
        std::memcpy(dst.data() + off_elems * 4, &v, 4);
    }
}

trimul_status check_shape(const trimul_handle* h, int B, int N)
{
    if (B < 1) return fail(TRIMUL_ERR_INVALID_ARG, "B must be >= 1; got %d", B);
    if (N < 8 || N % 8 != 0)
        return fail(TRIMUL_ERR_INVALID_ARG, "N must be a multiple of 8 and >= 8 (16-byte rows); got %d", N);
    if (N > 32768) return fail(TRIMUL_ERR_UNSUPPORTED, "N must be <= 32768; got %d", N);
    if ((long long)B * h->p.C > 65535)
        return fail(TRIMUL_ERR_UNSUPPORTED, "B*C must be <= 65535; got %lld", (long long)B * h->p.C);
    // Every launch covers at most 2 threads per pair; keep that below 2^32.
    if ((long long)B * N * N >= (1LL << 31))
        return fail(TRIMUL_ERR_UNSUPPORTED, "B*N*N must be < 2^31; got %lld", (long long)B * N * N);
    return TRIMUL_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    if (!a || !b || !na || !nb) return false;
    uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// Per-device address of `scratch`, looked up once per device with that device
// current (the caller's), and kept for the life of the process.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];

trimul_status scratch_address(int dev, void** out)
{
    if (dev < 0 || dev >= kMaxDevices)
        return fail(TRIMUL_ERR_UNSUPPORTED, "device ordinal %d is beyond the %d the library tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail("hipGetSymbolAddress (scratch)", e);
        if (!ptr) return fail(TRIMUL_ERR_HIP, "hipGetSymbolAddress (scratch) returned NULL");
        g_scratch_addr[dev] = ptr;
    }
    *out = g_scratch_addr[dev];
    return TRIMUL_OK;
}

trimul_status check_handle_device(const trimul_handle* h)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    if (dev != h->device)
        return fail(TRIMUL_ERR_INVALID_ARG, "handle was created on device %d but device %d is current",
                    h->device, dev);
    return TRIMUL_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// The integer a C caller passed for an enum argument.  C allows any int there,
// while in C++ merely loading an enum object that holds a value outside the
// enum's range is undefined, so the value is read as its object
// representation and only validated ints are turned back into enums.
template <typename E>
int enum_int(const E* e)
{
    static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
    int v;
    std::memcpy(&v, e, sizeof v);
    return v;
}

bool direction_ok(int d) { return d == TRIMUL_OUTGOING || d == TRIMUL_INCOMING; }

int device_cus()
{
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    return cus;
}

// Workspace carving.  Full layout: a | b | o | mask table.  Lean layout: a | b |
// spare | mask table, where the contraction runs in chunks of `chunk` slabs: the
// first chunk's o goes to the spare region, chunk t's o over the a slabs of
// chunk t - 1 (which chunk t - 1 has finished reading; stream order), so o
// needs only one chunk of memory of its own.  chunk is the smallest multiple
// of 8 slabs that gives every workgroup of a persistent launch at least 8
// tiles (8 * 256 tiles), at most all B*C slabs.
struct WsLayout {
    size_t a, b, o, ranges, total;   // byte offsets and size
    int chunk;                       // slabs per contraction launch (B*C when not lean)
    bool lean;
};

WsLayout ws_layout(int C, trimul_dtype dt, int B, int N, bool lean)
{
    const trimul::DType t = dt == TRIMUL_BF16 ? trimul::DType::BF16 : trimul::DType::FP32;
    const size_t es = elem_size(dt), NN = (size_t)N * N;
    const int nbc = B * C;
    WsLayout L;
    L.lean = lean;
    L.chunk = nbc;
    if (lean) {
        const long long tiles = (N + trimul::K2_TILE - 1) / trimul::K2_TILE;
        const long long want = 8LL * 256;
        long long ch = 8;
        while (ch < nbc && ch * tiles * tiles < want) ch += 8;
        L.chunk = (int)(ch < nbc ? ch : nbc);
    }
    const size_t ab = align256((size_t)nbc * trimul::ab_slab_elems(t, N) * es);
    const size_t ob = align256((size_t)L.chunk * NN * es);
    const size_t rb = align256(trimul::mask_table_ints(B, N) * sizeof(int));
    L.a = 0;
    L.b = ab;
    L.o = 2 * ab;
    L.ranges = L.o + ob;
    L.total = L.ranges + rb;
    return L;
}

// One validated forward call.
struct FwdCall {
    const void* z;
    const void* mask;
    int B, N, incoming;
    void* out;
    uint8_t* ws;
    WsLayout L;
};

trimul::PlanKey key_of(const FwdCall& c) { return {c.B, c.N, c.incoming, c.mask ? 1 : 0}; }

trimul::Plan plan_lookup(trimul_handle* h, const trimul::PlanKey& k)
{
    std::lock_guard<std::mutex> g(h->mu);
    for (const trimul::PlanEntry& e : h->plans)
        if (e.key == k) return e.plan;
    return trimul::default_plan(k);
}

trimul::Plan plan_for(trimul_handle* h, const FwdCall& c) { return plan_lookup(h, key_of(c)); }

void set_plan(trimul_handle* h, const trimul::PlanEntry& ent)
{
    std::lock_guard<std::mutex> g(h->mu);
    for (trimul::PlanEntry& e : h->plans)
        if (e.key == ent.key) {
            e = ent;
            return;
        }
    h->plans.push_back(ent);
}

// Every check of trimul_fwd, before anything is enqueued.  The workspace
// layout is the full one when the workspace holds it, else the lean one.
trimul_status prepare_fwd(trimul_handle* h, const void* z, const void* pair_mask, int B, int N,
                          trimul_direction dir, void* out, void* workspace, size_t workspace_bytes,
                          FwdCall& c)
{
    if (!h) return fail(TRIMUL_ERR_INVALID_ARG, "handle is NULL");
    if (!z) return fail(TRIMUL_ERR_INVALID_ARG, "z is NULL");
    if (!out) return fail(TRIMUL_ERR_INVALID_ARG, "out is NULL");
    const int d = enum_int(&dir);
    if (!direction_ok(d))
        return fail(TRIMUL_ERR_INVALID_ARG, "direction must be TRIMUL_OUTGOING or TRIMUL_INCOMING; got %d", d);
    trimul_status st = check_shape(h, B, N);
    if (st != TRIMUL_OK) return st;
    const trimul_dtype dt = (trimul_dtype)h->p.dtype;
    const size_t es = elem_size(dt);
    if (!aligned(z, 16)) return fail(TRIMUL_ERR_INVALID_ARG, "z must be 16-byte aligned");
    if (!aligned(out, 16)) return fail(TRIMUL_ERR_INVALID_ARG, "out must be 16-byte aligned");
    if (pair_mask && !aligned(pair_mask, 16)) return fail(TRIMUL_ERR_INVALID_ARG, "pair_mask must be 16-byte aligned");
    const WsLayout full = ws_layout(h->p.C, dt, B, N, false);
    const WsLayout lean = ws_layout(h->p.C, dt, B, N, true);
    if (!workspace)
        return fail(TRIMUL_ERR_WORKSPACE, "workspace is NULL (%zu bytes required, %zu with the lean layout)",
                    full.total, lean.total);
    if (workspace_bytes < lean.total)
        return fail(TRIMUL_ERR_WORKSPACE,
                    "workspace of %zu bytes is smaller than the %zu required (%zu with the lean layout)",
                    workspace_bytes, full.total, lean.total);
    if (!aligned(workspace, 256)) return fail(TRIMUL_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    c.L = workspace_bytes >= full.total ? full : lean;
    const size_t need = c.L.total;
    const size_t NN = (size_t)N * N;
    const size_t zbytes = (size_t)B * NN * h->p.D * es;
    const size_t mbytes = pair_mask ? (size_t)B * NN * es : 0;
    if (overlaps(out, zbytes, z, zbytes)) return fail(TRIMUL_ERR_INVALID_ARG, "out overlaps z");
    if (overlaps(out, zbytes, pair_mask, mbytes)) return fail(TRIMUL_ERR_INVALID_ARG, "out overlaps pair_mask");
    if (overlaps(out, zbytes, workspace, need)) return fail(TRIMUL_ERR_INVALID_ARG, "out overlaps the workspace");
    if (overlaps(z, zbytes, workspace, need)) return fail(TRIMUL_ERR_INVALID_ARG, "z overlaps the workspace");
    if (overlaps(pair_mask, mbytes, workspace, need))
        return fail(TRIMUL_ERR_INVALID_ARG, "pair_mask overlaps the workspace");
    st = check_handle_device(h);
    if (st != TRIMUL_OK) return st;
    c.z = z;
    c.mask = pair_mask;
    c.B = B;
    c.N = N;
    c.incoming = d == TRIMUL_INCOMING;
    c.out = out;
    c.ws = static_cast<uint8_t*>(workspace);
    return TRIMUL_OK;
}

bool uses_ranges(const trimul_handle* h, const FwdCall& c)
{
    return c.mask && h->p.dtype == trimul::DType::BF16;
}

// The mask scan (masked bf16 calls) and the projection.
hipError_t enq_project(const trimul_handle* h, const trimul::Plan& plan, const FwdCall& c, hipStream_t s)
{
    hipError_t e = hipSuccess;
    if (uses_ranges(h, c))
        e = trimul::launch_mask_ranges(h->p, c.mask, c.B, c.N, c.incoming, (int*)(c.ws + c.L.ranges), s);
    if (e == hipSuccess)
        e = trimul::launch_project(h->p, plan, c.z, c.mask, c.B, c.N, c.incoming, c.ws + c.L.a, c.ws + c.L.b, s);
    return e;
}

size_t ab_slab_bytes(const trimul_handle* h, int N)
{
    return trimul::ab_slab_elems(h->p.dtype, N) * elem_size((trimul_dtype)h->p.dtype);
}

// The contraction (after the pair lists of a masked call), in one launch or
// (lean layout) one launch per chunk.
hipError_t enq_contract(const trimul_handle* h, const trimul::Plan& plan, const FwdCall& c, hipStream_t s)
{
    const int nbc = c.B * h->p.C;
    const size_t es = elem_size((trimul_dtype)h->p.dtype), slab = ab_slab_bytes(h, c.N);
    int* table = uses_ranges(h, c) ? (int*)(c.ws + c.L.ranges) : nullptr;
    hipError_t e = table ? trimul::launch_tile_pairs(plan, table, c.B, c.N, s) : hipSuccess;
    for (int bc0 = 0; bc0 < nbc && e == hipSuccess; bc0 += c.L.chunk) {
        trimul::ContractJob job;
        job.bc0 = bc0;
        job.nbc = std::min(c.L.chunk, nbc - bc0);
        if (bc0 == 0) {
            job.o = c.ws + c.L.o;
            job.o_stride = (size_t)c.N * c.N;
        } else {
            job.o = c.ws + c.L.a + (size_t)(bc0 - c.L.chunk) * slab;
            job.o_stride = slab / es;
        }
        job.table = table;
        e = trimul::launch_contract(h->p, plan, c.ws + c.L.a, c.ws + c.L.b, c.B, c.N, job, s);
    }
    return e;
}

hipError_t enq_output(const trimul_handle* h, const FwdCall& c, hipStream_t s)
{
    trimul::OutputSrc os;
    os.o_lo = c.ws + c.L.o;
    os.o_hi = c.ws + c.L.a;
    os.split = c.L.chunk;
    os.hi_stride = ab_slab_bytes(h, c.N) / elem_size((trimul_dtype)h->p.dtype);
    return trimul::launch_output(h->p, c.z, os, c.B, c.N, c.out, s);
}

trimul_status enqueue_fwd(const trimul_handle* h, const trimul::Plan& plan, const FwdCall& c, hipStream_t s)
{
    hipError_t e = enq_project(h, plan, c, s);
    if (e != hipSuccess) return hip_fail("projection kernel launch", e);
    e = enq_contract(h, plan, c, s);
    if (e != hipSuccess) return hip_fail("contraction kernel launch", e);
    e = enq_output(h, c, s);
    if (e != hipSuccess) return hip_fail("output kernel launch", e);
    return ok();
}

}  // namespace

extern "C" {

const char* trimul_status_string(trimul_status s)
{
    switch (enum_int(&s)) {
    case TRIMUL_OK: return "TRIMUL_OK";
    case TRIMUL_ERR_INVALID_ARG: return "TRIMUL_ERR_INVALID_ARG";
    case TRIMUL_ERR_UNSUPPORTED: return "TRIMUL_ERR_UNSUPPORTED";
    case TRIMUL_ERR_ARCH: return "TRIMUL_ERR_ARCH";
    case TRIMUL_ERR_WORKSPACE: return "TRIMUL_ERR_WORKSPACE";
    case TRIMUL_ERR_HIP: return "TRIMUL_ERR_HIP";
    }
    return "TRIMUL_ERR_UNKNOWN";
}

const char* trimul_last_error(void) { return g_err; }

trimul_status trimul_check_arch(const char* name)
{
    if (!name) return fail(TRIMUL_ERR_INVALID_ARG, "architecture name is NULL");
    if (std::strncmp(name, "gfx950", 6) == 0 && (name[6] == '\0' || name[6] == ':')) return ok();
    return fail(TRIMUL_ERR_ARCH, "libtrimul requires gfx950 (MI355X); got %s", name);
}

trimul_status trimul_workspace_query(int D, int C, trimul_dtype dtype, int B, int N, size_t* bytes)
{
    if (!bytes) return fail(TRIMUL_ERR_INVALID_ARG, "bytes is NULL");
    const int dt = enum_int(&dtype);
    if (dt != TRIMUL_BF16 && dt != TRIMUL_FP32)
        return fail(TRIMUL_ERR_INVALID_ARG, "dtype must be TRIMUL_BF16 or TRIMUL_FP32; got %d", dt);
    if (!width_ok(D) || !width_ok(C))
        return fail(TRIMUL_ERR_UNSUPPORTED, "D and C must be multiples of 32 in [32, 256]; got D=%d C=%d", D, C);
    if (B < 1 || N < 1) return fail(TRIMUL_ERR_INVALID_ARG, "B and N must be >= 1; got B=%d N=%d", B, N);
    *bytes = ws_layout(C, (trimul_dtype)dt, B, N, false).total;
    return ok();
}

trimul_status trimul_workspace_size(const trimul_handle* h, int B, int N, size_t* bytes)
{
    if (!h) return fail(TRIMUL_ERR_INVALID_ARG, "handle is NULL");
    return trimul_workspace_query(h->p.D, h->p.C, (trimul_dtype)h->p.dtype, B, N, bytes);
}

trimul_status trimul_workspace_size_lean(const trimul_handle* h, int B, int N, size_t* bytes)
{
    if (!h) return fail(TRIMUL_ERR_INVALID_ARG, "handle is NULL");
    if (!bytes) return fail(TRIMUL_ERR_INVALID_ARG, "bytes is NULL");
    if (B < 1 || N < 1) return fail(TRIMUL_ERR_INVALID_ARG, "B and N must be >= 1; got B=%d N=%d", B, N);
    *bytes = ws_layout(h->p.C, (trimul_dtype)h->p.dtype, B, N, true).total;
    return ok();
}

trimul_status trimul_create(int D, int C, trimul_dtype dtype_arg, const trimul_weights* w,
                            trimul_handle** out)
{
    return guarded([&]() -> trimul_status {
        if (!out) return fail(TRIMUL_ERR_INVALID_ARG, "out (handle pointer) is NULL");
        *out = nullptr;
        if (!w) return fail(TRIMUL_ERR_INVALID_ARG, "weights is NULL");
        const int dt = enum_int(&dtype_arg);
        if (dt != TRIMUL_BF16 && dt != TRIMUL_FP32)
            return fail(TRIMUL_ERR_INVALID_ARG, "dtype must be TRIMUL_BF16 or TRIMUL_FP32; got %d", dt);
        const trimul_dtype dtype = (trimul_dtype)dt;
        if (!width_ok(D) || !width_ok(C))
            return fail(TRIMUL_ERR_UNSUPPORTED, "D and C must be multiples of 32 in [32, 256]; got D=%d C=%d", D, C);
        const struct { const float* p; const char* n; } req[] = {
            {w->norm_in_weight, "norm_in_weight"}, {w->norm_in_bias, "norm_in_bias"},
            {w->p_in, "p_in"}, {w->g_in, "g_in"}, {w->norm_out_weight, "norm_out_weight"},
            {w->norm_out_bias, "norm_out_bias"}, {w->p_out, "p_out"}, {w->g_out, "g_out"}};
        for (const auto& r : req)
            if (!r.p) return fail(TRIMUL_ERR_INVALID_ARG, "weights->%s is NULL", r.n);
        if (!(w->eps > 0.0f) || !std::isfinite(w->eps))
            return fail(TRIMUL_ERR_INVALID_ARG, "eps must be finite and > 0; got %g", (double)w->eps);

        int dev = -1;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return hip_fail("hipGetDevice", e);
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail("hipGetDeviceProperties", e);
        trimul_status st = trimul_check_arch(prop.gcnArchName);
        if (st != TRIMUL_OK) return st;
        void* scratch_ptr = nullptr;
        st = scratch_address(dev, &scratch_ptr);
        if (st != TRIMUL_OK) return st;

        // Host packing.
        const size_t es = elem_size(dtype);
        const size_t n_proj = (size_t)4 * C * D, n_go = (size_t)D * D, n_po = (size_t)D * C;
        const size_t off_proj = 0;
        const size_t off_go = align256(n_proj * es);
        const size_t off_po = off_go + align256(n_go * es);
        const size_t off_ln = off_po + align256(n_po * es);
        const size_t off_gof = off_ln + align256((size_t)(2 * D + 2 * C) * 4);
        const bool folded = dtype == TRIMUL_BF16;
        const size_t off_pof = off_gof + (folded ? align256(n_go * 2) : 0);
        const size_t off_xg = off_pof + (folded ? align256(n_po * 2) : 0);
        const size_t off_xp = off_xg + (folded ? align256((size_t)D * 16) : 0);
        const size_t off_wpf = off_xp + (folded ? align256((size_t)D * 16) : 0);
        const size_t off_xpj = off_wpf + (folded ? align256(n_proj * 2) : 0);
        const size_t off_sink = off_xpj + (folded ? align256((size_t)4 * C * 16) : 0);
        const size_t total = off_sink + 4096;
        std::vector<uint8_t> host(total, 0);
        if (folded) {
            fold_rows(w->g_out, w->norm_in_weight, w->norm_in_bias, D, D,
                      reinterpret_cast<uint16_t*>(host.data() + off_gof),
                      reinterpret_cast<uint16_t*>(host.data() + off_xg));
            fold_rows(w->p_out, w->norm_out_weight, w->norm_out_bias, D, C,
                      reinterpret_cast<uint16_t*>(host.data() + off_pof),
                      reinterpret_cast<uint16_t*>(host.data() + off_xp));
        }
        {
            std::vector<uint8_t> go(n_go * es), po(n_po * es);
            // Projection rows in the kernels' order: for a then b, per 16-channel
            // group, 16 rows of p_in then the same channels' 16 rows of g_in.
            std::vector<float> projf(n_proj);
            size_t row = 0;
            for (int part = 0; part < 2; ++part)          // a, then b
                for (int g = 0; g < C / 16; ++g) {        // 16-channel groups
                    for (int r = 0; r < 16; ++r, ++row)   // p rows
                        std::memcpy(&projf[row * D], w->p_in + ((size_t)part * C + g * 16 + r) * D, D * 4);
                    for (int r = 0; r < 16; ++r, ++row)   // g rows of the same channels
                        std::memcpy(&projf[row * D], w->g_in + ((size_t)part * C + g * 16 + r) * D, D * 4);
                }
            std::vector<uint8_t> proj(n_proj * es);
            for (size_t i = 0; i < n_proj; ++i) put(proj, i, projf[i], dtype);
            if (folded)
                fold_projection_rows(projf.data(), w->norm_in_weight, w->norm_in_bias, 4 * C, D,
                                     reinterpret_cast<uint16_t*>(host.data() + off_wpf),
                                     reinterpret_cast<float*>(host.data() + off_xpj));
            for (size_t i = 0; i < n_go; ++i) put(go, i, w->g_out[i], dtype);
            for (size_t i = 0; i < n_po; ++i) put(po, i, w->p_out[i], dtype);
            std::memcpy(host.data() + off_proj, proj.data(), proj.size());
            std::memcpy(host.data() + off_go, go.data(), go.size());
            std::memcpy(host.data() + off_po, po.data(), po.size());
            float* ln = reinterpret_cast<float*>(host.data() + off_ln);
            std::memcpy(ln, w->norm_in_weight, D * 4);
            std::memcpy(ln + D, w->norm_in_bias, D * 4);
            std::memcpy(ln + 2 * D, w->norm_out_weight, C * 4);
            std::memcpy(ln + 2 * D + C, w->norm_out_bias, C * 4);
        }

        // Everything that can throw happens before the device allocation: the
        // device key, and the plans recorded by trimul_tune in an earlier
        // process (an unreadable cache only means no recorded plans).
        std::string arch = trimul::plan_device_key(prop.gcnArchName, prop.multiProcessorCount);
        std::vector<trimul::PlanEntry> plans;
        (void)trimul::plan_cache_load(trimul::plan_cache_path(), arch, D, C, (int)dtype, plans);

        void* mem = nullptr;
        e = hipMalloc(&mem, total);
        if (e != hipSuccess) return hip_fail("hipMalloc (packed weights)", e);
        e = hipMemcpy(mem, host.data(), total, hipMemcpyHostToDevice);
        if (e != hipSuccess) {
            (void)hipFree(mem);
            return hip_fail("hipMemcpy (packed weights)", e);
        }
        trimul_handle* h = new (std::nothrow) trimul_handle;
        if (!h) {
            (void)hipFree(mem);
            return fail(TRIMUL_ERR_INVALID_ARG, "out of host memory");
        }
        uint8_t* base = static_cast<uint8_t*>(mem);
        h->dev_mem = mem;
        h->device = dev;
        h->p.D = D;
        h->p.C = C;
        h->p.dtype = dtype == TRIMUL_BF16 ? trimul::DType::BF16 : trimul::DType::FP32;
        h->p.eps = w->eps;
        h->p.w_proj = base + off_proj;
        h->p.w_gout = base + off_go;
        h->p.w_pout = base + off_po;
        const float* ln = reinterpret_cast<const float*>(base + off_ln);
        h->p.ln_in_w = ln;
        h->p.ln_in_b = ln + D;
        h->p.ln_out_w = ln + 2 * D;
        h->p.ln_out_b = ln + 2 * D + C;
        h->p.w_gout_f = folded ? base + off_gof : nullptr;
        h->p.w_pout_f = folded ? base + off_pof : nullptr;
        h->p.x_gout = folded ? base + off_xg : nullptr;
        h->p.x_pout = folded ? base + off_xp : nullptr;
        h->p.w_proj_f = folded ? base + off_wpf : nullptr;
        h->p.x_proj = folded ? base + off_xpj : nullptr;
        h->p.sink = base + off_sink;
        h->scratch = scratch_ptr;
        h->arch = std::move(arch);
        h->plans = std::move(plans);
        *out = h;
        return ok();
    });
}

void trimul_destroy(trimul_handle* h)
{
    if (!h) return;
    if (h->dev_mem) (void)hipFree(h->dev_mem);
    delete h;
}

trimul_status trimul_fwd(trimul_handle* h, const void* z, const void* pair_mask, int B, int N,
                         trimul_direction dir, void* out, void* workspace, size_t workspace_bytes,
                         hipStream_t stream)
{
    FwdCall c;
    trimul_status st = prepare_fwd(h, z, pair_mask, B, N, dir, out, workspace, workspace_bytes, c);
    if (st != TRIMUL_OK) return st;
    return enqueue_fwd(h, plan_for(h, c), c, stream);
}

trimul_status trimul_fwd_noalloc(trimul_handle* h, const void* z, const void* pair_mask, int B, int N,
                                 trimul_direction dir, void* out, hipStream_t stream)
{
    if (!h) return fail(TRIMUL_ERR_INVALID_ARG, "handle is NULL");
    trimul_status st = check_shape(h, B, N);
    if (st != TRIMUL_OK) return st;
    const trimul_dtype dt = (trimul_dtype)h->p.dtype;
    const size_t need = ws_layout(h->p.C, dt, B, N, true).total;
    if (need > (size_t)TRIMUL_NOALLOC_MAX_BYTES)
        return fail(TRIMUL_ERR_UNSUPPORTED,
                    "B=%d N=%d needs %zu bytes of scratch (lean layout); trimul_fwd_noalloc holds %zu: "
                    "use trimul_fwd with a workspace", B, N, need, (size_t)TRIMUL_NOALLOC_MAX_BYTES);
    FwdCall c;
    st = prepare_fwd(h, z, pair_mask, B, N, dir, out, h->scratch, (size_t)TRIMUL_NOALLOC_MAX_BYTES, c);
    if (st != TRIMUL_OK) return st;
    return enqueue_fwd(h, plan_for(h, c), c, stream);
}

trimul_status trimul_tune(trimul_handle* h, const void* z, const void* pair_mask, int B, int N,
                          trimul_direction dir, void* out, void* workspace, size_t workspace_bytes,
                          hipStream_t stream)
{
    return guarded([&]() -> trimul_status {
        FwdCall c;
        trimul_status st = prepare_fwd(h, z, pair_mask, B, N, dir, out, workspace, workspace_bytes, c);
        if (st != TRIMUL_OK) return st;
        hipEvent_t e0 = nullptr, e1 = nullptr;
        hipError_t e = hipEventCreate(&e0);
        if (e == hipSuccess) e = hipEventCreate(&e1);
        if (e != hipSuccess) {
            if (e0) (void)hipEventDestroy(e0);
            return hip_fail("hipEventCreate", e);
        }
        // The projection variants, each timed between two events (its output
        // is the same for every variant), then the contraction choices, each
        // after a fresh projection (the lean layout overwrites a while the
        // contraction runs); one untimed warm-up, then the best of kReps.
        constexpr int kReps = 3;
        auto time_best = [&](auto&& before, auto&& timed, double& t_min) {
            t_min = 1e300;
            for (int r = 0; r <= kReps && e == hipSuccess; ++r) {
                e = before();
                if (e == hipSuccess) e = hipEventRecord(e0, stream);
                if (e == hipSuccess) e = timed();
                if (e == hipSuccess) e = hipEventRecord(e1, stream);
                if (e == hipSuccess) e = hipEventSynchronize(e1);
                float ms = 0.f;
                if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
                if (e == hipSuccess && r > 0 && ms < t_min) t_min = ms;
            }
        };
        trimul::Plan best;
        double best_k1 = 1e300, best_k2 = 1e300;
        for (int v : trimul::k1_variants()) {
            trimul::Plan pl = best;
            pl.k1_variant = v;
            double t;
            time_best([&]() { return hipSuccess; }, [&]() { return enq_project(h, pl, c, stream); }, t);
            if (e != hipSuccess) break;
            if (t < best_k1) { best_k1 = t; best.k1_variant = v; }
        }
        for (const trimul::Plan& k2 : trimul::k2_choices()) {
            if (e != hipSuccess) break;
            trimul::Plan pl = best;
            pl.k2_order = k2.k2_order;
            pl.k2_gm = k2.k2_gm;
            pl.k2_tile = k2.k2_tile;
            double t;
            time_best([&]() { return enq_project(h, pl, c, stream); }, [&]() { return enq_contract(h, pl, c, stream); },
                      t);
            if (e != hipSuccess) break;
            if (t < best_k2) {
                best_k2 = t;
                best.k2_order = pl.k2_order;
                best.k2_gm = pl.k2_gm;
                best.k2_tile = pl.k2_tile;
            }
        }
        const double best_ms = best_k1 + best_k2;
        (void)hipEventDestroy(e0);
        (void)hipEventDestroy(e1);
        if (e != hipSuccess) return hip_fail("tuning run", e);
        trimul::PlanEntry ent;
        ent.key = key_of(c);
        ent.plan = best;
        ent.ms = best_ms;
        set_plan(h, ent);
        // The cache is best effort: a read-only or missing location only means the
        // next process tunes again.
        try {
            (void)trimul::plan_cache_store(trimul::plan_cache_path(), h->arch, h->p.D, h->p.C, (int)h->p.dtype,
                                           ent);
        } catch (...) {
        }
        // Leave a correct result in out, computed with the chosen plan.
        return enqueue_fwd(h, best, c, stream);
    });
}

trimul_status trimul_internal_project(trimul_handle* h, const void* z, const void* pair_mask, int B,
                                      int N, trimul_direction dir, void* a_cm, void* b_cm,
                                      hipStream_t stream)
{
    if (!h) return fail(TRIMUL_ERR_INVALID_ARG, "handle is NULL");
    if (!z || !a_cm || !b_cm) return fail(TRIMUL_ERR_INVALID_ARG, "z, a_cm and b_cm must be non-NULL");
    const int d = enum_int(&dir);
    if (!direction_ok(d))
        return fail(TRIMUL_ERR_INVALID_ARG, "direction must be TRIMUL_OUTGOING or TRIMUL_INCOMING; got %d", d);
    trimul_status st = check_shape(h, B, N);
    if (st != TRIMUL_OK) return st;
    if (!aligned(z, 16) || !aligned(a_cm, 16) || !aligned(b_cm, 16))
        return fail(TRIMUL_ERR_INVALID_ARG, "z, a_cm and b_cm must be 16-byte aligned");
    if (pair_mask && !aligned(pair_mask, 16)) return fail(TRIMUL_ERR_INVALID_ARG, "pair_mask must be 16-byte aligned");
    st = check_handle_device(h);
    if (st != TRIMUL_OK) return st;
    const trimul::Plan plan = plan_lookup(h, {B, N, d, pair_mask ? 1 : 0});
    hipError_t e = trimul::launch_project(h->p, plan, z, pair_mask, B, N, d == TRIMUL_INCOMING, a_cm, b_cm, stream);
    if (e != hipSuccess) return hip_fail("projection kernel launch", e);
    return ok();
}

trimul_status trimul_internal_mask_ranges(trimul_handle* h, const void* pair_mask, int B, int N,
                                          trimul_direction dir, int* table, hipStream_t stream)
{
    if (!h) return fail(TRIMUL_ERR_INVALID_ARG, "handle is NULL");
    if (!pair_mask || !table) return fail(TRIMUL_ERR_INVALID_ARG, "pair_mask and table must be non-NULL");
    const int d = enum_int(&dir);
    if (!direction_ok(d))
        return fail(TRIMUL_ERR_INVALID_ARG, "direction must be TRIMUL_OUTGOING or TRIMUL_INCOMING; got %d", d);
    trimul_status st = check_shape(h, B, N);
    if (st != TRIMUL_OK) return st;
    if (!aligned(pair_mask, 16) || !aligned(table, 16))
        return fail(TRIMUL_ERR_INVALID_ARG, "pair_mask and table must be 16-byte aligned");
    st = check_handle_device(h);
    if (st != TRIMUL_OK) return st;
    hipError_t e = trimul::launch_mask_ranges(h->p, pair_mask, B, N, d == TRIMUL_INCOMING, table, stream);
    if (e != hipSuccess) return hip_fail("mask range kernel launch", e);
    return ok();
}

trimul_status trimul_internal_contract(trimul_handle* h, const void* a_cm, const void* b_cm, int* table,
                                       int B, int N, trimul_direction dir, void* o, hipStream_t stream)
{
    if (!h) return fail(TRIMUL_ERR_INVALID_ARG, "handle is NULL");
    if (!a_cm || !b_cm || !o) return fail(TRIMUL_ERR_INVALID_ARG, "a_cm, b_cm and o must be non-NULL");
    trimul_status st = check_shape(h, B, N);
    if (st != TRIMUL_OK) return st;
    if (!aligned(a_cm, 16) || !aligned(b_cm, 16) || !aligned(o, 16))
        return fail(TRIMUL_ERR_INVALID_ARG, "a_cm, b_cm and o must be 16-byte aligned");
    const int d = enum_int(&dir);
    if (!direction_ok(d))
        return fail(TRIMUL_ERR_INVALID_ARG, "direction must be TRIMUL_OUTGOING or TRIMUL_INCOMING; got %d", d);
    if (table && h->p.dtype != trimul::DType::BF16)
        return fail(TRIMUL_ERR_UNSUPPORTED, "the mask table is used by the bf16 contraction only");
    if (table && !aligned(table, 16)) return fail(TRIMUL_ERR_INVALID_ARG, "table must be 16-byte aligned");
    st = check_handle_device(h);
    if (st != TRIMUL_OK) return st;
    const trimul::Plan plan = plan_lookup(h, {B, N, d, table ? 1 : 0});
    trimul::ContractJob job;
    job.bc0 = 0;
    job.nbc = B * h->p.C;
    job.o = o;
    job.o_stride = (size_t)N * N;
    job.table = table;
    hipError_t e = table ? trimul::launch_tile_pairs(plan, table, B, N, stream) : hipSuccess;
    if (e == hipSuccess) e = trimul::launch_contract(h->p, plan, a_cm, b_cm, B, N, job, stream);
    if (e != hipSuccess) return hip_fail("contraction kernel launch", e);
    return ok();
}

trimul_status trimul_internal_output(trimul_handle* h, const void* z, const void* o, int B, int N,
                                     void* out, hipStream_t stream)
{
    if (!h) return fail(TRIMUL_ERR_INVALID_ARG, "handle is NULL");
    if (!z || !o || !out) return fail(TRIMUL_ERR_INVALID_ARG, "z, o and out must be non-NULL");
    trimul_status st = check_shape(h, B, N);
    if (st != TRIMUL_OK) return st;
    if (!aligned(z, 16) || !aligned(o, 16) || !aligned(out, 16))
        return fail(TRIMUL_ERR_INVALID_ARG, "z, o and out must be 16-byte aligned");
    st = check_handle_device(h);
    if (st != TRIMUL_OK) return st;
    trimul::OutputSrc os;
    os.o_lo = o;
    os.o_hi = o;
    os.split = B * h->p.C;
    os.hi_stride = 0;
    hipError_t e = trimul::launch_output(h->p, z, os, B, N, out, stream);
    if (e != hipSuccess) return hip_fail("output kernel launch", e);
    return ok();
}

trimul_status trimul_internal_peak_mfma(const void* seed, int blocks, int iters, int shape, float* sink,
                                        hipStream_t stream)
{
    if (!seed || !sink) return fail(TRIMUL_ERR_INVALID_ARG, "seed and sink must be non-NULL");
    if (!aligned(seed, 16) || !aligned(sink, 4))
        return fail(TRIMUL_ERR_INVALID_ARG, "seed must be 16-byte aligned and sink 4-byte aligned");
    if (blocks < 1 || blocks > (1 << 20)) return fail(TRIMUL_ERR_INVALID_ARG, "blocks must be in [1, 2^20]; got %d", blocks);
    if (iters < 1 || iters > (1 << 24)) return fail(TRIMUL_ERR_INVALID_ARG, "iters must be in [1, 2^24]; got %d", iters);
    if (shape != 0 && shape != 1) return fail(TRIMUL_ERR_INVALID_ARG, "shape must be 0 or 1; got %d", shape);
    hipError_t e = trimul::launch_peak_mfma(seed, blocks, iters, shape, sink, stream);
    if (e != hipSuccess) return hip_fail("MFMA peak kernel launch", e);
    return ok();
}

trimul_status trimul_internal_peak_stream(const void* src0, const void* src1, void* dst0, void* dst1, size_t n16,
                                          int reads, int writes, int nontemporal, hipStream_t stream)
{
    if (!((reads == 1 && writes == 1) || (reads == 2 && writes == 1) || (reads == 1 && writes == 2)))
        return fail(TRIMUL_ERR_INVALID_ARG, "(reads, writes) must be (1, 1), (2, 1) or (1, 2); got (%d, %d)", reads, writes);
    if (n16 < 1 || n16 > ((size_t)1 << 38)) return fail(TRIMUL_ERR_INVALID_ARG, "n16 must be in [1, 2^38]");
    if (!src0 || !dst0 || (reads == 2 && !src1) || (writes == 2 && !dst1))
        return fail(TRIMUL_ERR_INVALID_ARG, "a buffer the mode uses is NULL");
    if (!aligned(src0, 16) || !aligned(dst0, 16) || (reads == 2 && !aligned(src1, 16)) ||
        (writes == 2 && !aligned(dst1, 16)))
        return fail(TRIMUL_ERR_INVALID_ARG, "stream buffers must be 16-byte aligned");
    hipError_t e = trimul::launch_peak_stream(src0, src1, dst0, dst1, n16, reads, writes, nontemporal, stream);
    if (e != hipSuccess) return hip_fail("stream peak kernel launch", e);
    return ok();
}

trimul_status trimul_internal_set_plan(trimul_handle* h, int B, int N, trimul_direction dir, int masked,
                                       int k1_variant, int k2_order, int k2_gm, int k2_tile)
{
    return guarded([&]() -> trimul_status {
        if (!h) return fail(TRIMUL_ERR_INVALID_ARG, "handle is NULL");
        trimul::PlanEntry ent;
        ent.key = {B, N, enum_int(&dir), masked ? 1 : 0};
        ent.plan.k1_variant = k1_variant;
        ent.plan.k2_order = k2_order;
        ent.plan.k2_gm = k2_gm;
        ent.plan.k2_tile = k2_tile;
        ent.ms = 0.0;
        if (!trimul::plan_valid(ent.plan))
            return fail(TRIMUL_ERR_INVALID_ARG, "no candidate plan has k1_variant=%d k2_order=%d k2_gm=%d k2_tile=%d",
                        k1_variant, k2_order, k2_gm, k2_tile);
        set_plan(h, ent);
        return ok();
    });
}

trimul_status trimul_internal_get_plan(trimul_handle* h, int B, int N, trimul_direction dir, int masked,
                                       int* k1_variant, int* k2_order, int* k2_gm, int* k2_tile)
{
    return guarded([&]() -> trimul_status {
        if (!h || !k1_variant || !k2_order || !k2_gm || !k2_tile)
            return fail(TRIMUL_ERR_INVALID_ARG, "handle and outputs must be non-NULL");
        const trimul::Plan p = plan_lookup(h, {B, N, enum_int(&dir), masked ? 1 : 0});
        *k1_variant = p.k1_variant;
        *k2_order = p.k2_order;
        *k2_gm = p.k2_gm;
        *k2_tile = p.k2_tile;
        return ok();
    });
}

int trimul_internal_plan_candidates(int* k1_variant, int* k2_order, int* k2_gm, int* k2_tile, int cap)
{
    return guarded_int([&]() -> int {
        const std::vector<trimul::Plan> c = trimul::candidate_plans();
        for (int i = 0; i < (int)c.size() && i < cap; ++i) {
            if (k1_variant) k1_variant[i] = c[i].k1_variant;
            if (k2_order) k2_order[i] = c[i].k2_order;
            if (k2_gm) k2_gm[i] = c[i].k2_gm;
            if (k2_tile) k2_tile[i] = c[i].k2_tile;
        }
        return (int)c.size();
    }, -1);
}

trimul_status trimul_internal_cache_store(const char* path, const char* device, int D, int C, int dtype,
                                          int B, int N, int dir, int masked, int k1_variant, int k2_order,
                                          int k2_gm, int k2_tile, double ms)
{
    return guarded([&]() -> trimul_status {
        if (!path || !device) return fail(TRIMUL_ERR_INVALID_ARG, "path and device must be non-NULL");
        trimul::PlanEntry ent;
        ent.key = {B, N, dir, masked};
        ent.plan.k1_variant = k1_variant;
        ent.plan.k2_order = k2_order;
        ent.plan.k2_gm = k2_gm;
        ent.plan.k2_tile = k2_tile;
        ent.ms = ms;
        if (!trimul::plan_valid(ent.plan))
            return fail(TRIMUL_ERR_INVALID_ARG, "no candidate plan has k1_variant=%d k2_order=%d k2_gm=%d k2_tile=%d",
                        k1_variant, k2_order, k2_gm, k2_tile);
        if (!trimul::plan_cache_store(path, device, D, C, dtype, ent))
            return fail(TRIMUL_ERR_INVALID_ARG, "could not write the plan cache %s", path);
        return ok();
    });
}

int trimul_internal_cache_lookup(const char* path, const char* device, int D, int C, int dtype, int B, int N,
                                 int dir, int masked, int* k1_variant, int* k2_order, int* k2_gm,
                                 int* k2_tile)
{
    return guarded_int([&]() -> int {
        if (!path || !device) return -1;
        std::vector<trimul::PlanEntry> v;
        if (!trimul::plan_cache_load(path, device, D, C, dtype, v)) return -1;
        const trimul::PlanKey k = {B, N, dir, masked};
        for (const trimul::PlanEntry& e : v)
            if (e.key == k) {
                if (k1_variant) *k1_variant = e.plan.k1_variant;
                if (k2_order) *k2_order = e.plan.k2_order;
                if (k2_gm) *k2_gm = e.plan.k2_gm;
                if (k2_tile) *k2_tile = e.plan.k2_tile;
                return 1;
            }
        return 0;
    }, -1);
}

int trimul_internal_cache_path(char* buf, int cap)
{
    return guarded_int([&]() -> int {
        const std::string p = trimul::plan_cache_path();
        if (buf && cap > 0) {
            std::snprintf(buf, (size_t)cap, "%s", p.c_str());
        }
        return (int)p.size();
    }, 0);
}

}  // extern "C"
