// k2_contract.hip -- the triangle contraction: for every (batch, channel) slab,
// o[i][j] = sum_k a_cm[i][k] * b_cm[j][k] over k in [0, N), fp32 accumulation
// on matrix cores, one rounding to the storage type at the end.
//
// The projection kernel stores a and b channel-major with k contiguous for both
// directions (the incoming direction's transpose is folded into that store), so
// this is always an "NT" product of two K-contiguous operands.  fp32 operand
// slabs are plain [row][k]; bf16 slabs are K-blocked (kblk_off: blocks of 32 k
// holding all rows), so every K-step reads whole contiguous runs.  o is always
// plain [i][j].  bf16 runs the persistent kernel k2_contract_ppp at every N;
// fp32 the register-staged kernel k2_contract.
//
// k2_contract (fp32): a 256-thread workgroup (4 waves in a 2 x 2 grid) owns a BM x BN tile
// of o; each wave owns (BM/2) x (BN/2) as 16 x 16 MFMA blocks.  K advances 128
// bytes per stage (64 bf16 / 32 fp32), staged through double-buffered LDS with
// the chunk swizzle of trimul_device.hpp; global loads for stage k+1 are in
// flight while stage k is multiplied.  Rows or K chunks past N read as zero, and
// stores past N are skipped, so any N that is a multiple of 8 works.
#include "trimul_device.hpp"
#include "trimul_launch.hpp"

namespace trimul {

template <typename T, int BM, int BN>
__global__ __launch_bounds__(256) void k2_contract(const T* __restrict__ A, const T* __restrict__ Bm,
                                                   T* __restrict__ O, int N, int tiles_j)
{
    constexpr int CE = Elem<T>::CE;
    constexpr int KCH = 8;                  // 16-byte chunks per tile row per stage
    constexpr int BK = KCH * CE;            // K elements per stage
    constexpr int WM = BM / 2, WN = BN / 2; // wave tile
    constexpr int FM = WM / 16, FN = WN / 16;
    constexpr int A_LD = BM * KCH / 256;    // chunks each thread loads per stage
    constexpr int B_LD = BN * KCH / 256;
    __shared__ u32x4 lds[2][(BM + BN) * KCH];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const size_t slab = (size_t)N * N;
    // Tile order.  Workgroups are handed to the 8 XCDs round-robin by id, so id g
    // runs on XCD g % 8.  Give each XCD a contiguous range of logical tiles
    // (channel-major), and inside a channel walk groups of GM tile rows column by
    // column: the ~32 tiles an XCD runs at once then share GM row panels of a and
    // a few column panels of b in that XCD's L2.
    const int tiles_i = (N + BM - 1) / BM;
    const int per_bc = tiles_i * tiles_j;
    const unsigned total = gridDim.x;                 // B*C*per_bc, a multiple of 8
    const unsigned g = blockIdx.x;
    const unsigned logical = (g & 7u) * (total >> 3) + (g >> 3);
    const size_t bc = logical / per_bc;
    const int t = (int)(logical % per_bc);
    constexpr int GM = 4;
    const int group = t / (GM * tiles_j);
    const int first_i = group * GM;
    const int gm = min(GM, tiles_i - first_i);
    const int ti = first_i + (t % (GM * tiles_j)) % gm;
    const int tj = (t % (GM * tiles_j)) / gm;
    static_assert(sizeof(T) == 4, "bf16 operands are K-blocked and use k2_contract_ppp");
    const T* Ab = A + bc * slab;
    const T* Bb = Bm + bc * slab;
    T* Ob = O + bc * slab;
    auto opoff = [&](int row, int k) -> size_t { return (size_t)row * N + k; };
    const int i0 = ti * BM, j0 = tj * BN;

    u32x4 ra[A_LD], rb[B_LD];
    const u32x4 zero = {0u, 0u, 0u, 0u};

    auto gload = [&](int k0) {
#pragma unroll
        for (int it = 0; it < A_LD; ++it) {
            int q = tid + 256 * it, row = q >> 3, c = q & 7;
            int gi = i0 + row, gk = k0 + c * CE;
            ra[it] = (gi < N && gk < N) ? ld16(Ab + opoff(gi, gk)) : zero;
        }
#pragma unroll
        for (int it = 0; it < B_LD; ++it) {
            int q = tid + 256 * it, row = q >> 3, c = q & 7;
            int gj = j0 + row, gk = k0 + c * CE;
            rb[it] = (gj < N && gk < N) ? ld16(Bb + opoff(gj, gk)) : zero;
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int it = 0; it < A_LD; ++it) {
            int q = tid + 256 * it, row = q >> 3, c = q & 7;
            lds[buf][row * KCH + swz(row, c)] = ra[it];
        }
#pragma unroll
        for (int it = 0; it < B_LD; ++it) {
            int q = tid + 256 * it, row = q >> 3, c = q & 7;
            lds[buf][BM * KCH + row * KCH + swz(row, c)] = rb[it];
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int m = 0; m < FM; ++m)
#pragma unroll
        for (int n = 0; n < FN; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (N + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
        for (int kg = 0; kg < KCH / 4; ++kg) {
            const int c = kg * 4 + (lane >> 4);
            u32x4 fa[FM], fb[FN];
#pragma unroll
            for (int m = 0; m < FM; ++m) {
                int row = wm * WM + m * 16 + (lane & 15);
                fa[m] = lds[buf][row * KCH + swz(row, c)];
            }
#pragma unroll
            for (int n = 0; n < FN; ++n) {
                int row = wn * WN + n * 16 + (lane & 15);
                fb[n] = lds[buf][BM * KCH + row * KCH + swz(row, c)];
            }
            // Operands swapped (b rows as the MFMA's A): each lane's four results
            // are four consecutive j of one i, so the store is one 4-element run.
#pragma unroll
            for (int m = 0; m < FM; ++m)
#pragma unroll
                for (int n = 0; n < FN; ++n) acc[m][n] = Elem<T>::mma(fb[n], fa[m], acc[m][n]);
        }
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int m = 0; m < FM; ++m) {
        const int i = i0 + wm * WM + m * 16 + (lane & 15);
#pragma unroll
        for (int n = 0; n < FN; ++n) {
            const int j = j0 + wn * WN + n * 16 + 4 * (lane >> 4);
            if (i < N && j < N) Elem<T>::store4(Ob, (size_t)i * N + j, acc[m][n]);
        }
    }
}

// ---------------------------------------------------------------------------
// Large-N bf16 path: 256 x 256 tiles fed by LDS DMA.
//
// K advances 32 per step.  The operand rows of a step (64 bytes each, 256 rows
// of a and 256 of b = 32 KB) live in a ring of LDS slots filled by
// buffer_load ... lds (global -> LDS without registers).  K chunks past N and
// steps past the workgroup's last tile are pushed out of the buffer's range
// and read as zero, so the ring runs past the last step without tail code;
// tile rows past N read zeros or other rows' data, which reach only outputs
// that are not stored.
//
// LDS layout of one operand in one slot (256 rows x 4 chunks of 16 bytes):
// rows are paired into 128-byte lines, line L = row / 2 holds the 16-byte slot
// ((row % 2) * 4 + chunk) ^ (L % 8).  For the MFMA fragment read (lane l: row
// l % 16 of a 16-row block, chunk l / 16) this is free of LDS bank conflicts on
// gfx950 (measured: 4 cycles per ds_read_b128, the rate of a contiguous read),
// and each 1 KB DMA write is contiguous.
// The compiler does not order LDS DMA against ds_read, so every hand-off is an
// explicit s_waitcnt + s_barrier.
// ---------------------------------------------------------------------------
namespace k2big {
constexpr int BM = 256, BN = 256, BK = 32;
constexpr int ROWB = 64;                       // bytes of one operand row per step
constexpr int OPB = BM * ROWB;                 // bytes of one operand per slot (16 KB)
constexpr int STB = 2 * OPB;                   // bytes per slot (a and b)

__device__ inline int slot_off(int row, int chunk)
{
    const int L = row >> 1;
    return L * 128 + (((((row & 1) << 2) | chunk) ^ (L & 7)) << 4);
}
}  // namespace k2big

#define TRIMUL_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// Persistent kernel: one 512-thread workgroup per CU walks its tiles g, g + G,
// ... in an XCD-banded order (workgroup g runs on XCD g % 8, each XCD gets a
// compact band of tiles, walked in groups of GM row panels column by column,
// so the ~32 tiles an XCD runs at once share K-slices of a few panels in its
// L2; GM = 8 measured best against 1, 2, 4 and 16 at N = 4096).
//
// 8 waves in a 2 x 4 grid, each owning a 128 x 64 block of the tile (8 x 4
// MFMA tiles, 128 accumulators per lane); the two waves that share a SIMD
// (wave w and w + 4) run half a step apart ("ping-pong").  Each wave
// alternates a memory phase M_k (read step k's fragments from LDS, issue its
// share of step k+3's DMA) and a compute phase C_k (32 MFMAs); group 0 (waves
// 0-3) is one phase ahead of group 1 (waves 4-7), so in every phase one wave of
// each SIMD multiplies while the other loads, and phases are separated by one
// workgroup barrier.  Steps are numbered across the workgroup's tiles.
//
// Phase p: group 0 runs M_{p/2} (p even) or C_{(p-1)/2} (p odd); group 1 runs
// the same one phase later.  Invariants (NSP = 4 slots, DMA three steps ahead):
//  - step k's slot is read in phases 2k (group 0) and 2k+1 (group 1); every
//    wave's DMA share of step k was issued at least four phases earlier, and
//    before each barrier a wave waits until at most two of its steps are in
//    flight, so step k has landed for everyone when phase 2k starts;
//  - step k+3's DMA overwrites step k-1's slot, first in phase 2k, after the
//    barrier that ends phase 2k-1 where the last reader (group 1) finished; a
//    memory phase ends with lgkmcnt(0) so its reads are complete at that barrier.
// Group 1 takes one extra barrier at the start and group 0 one at the end, so
// every wave executes the same number of barriers.
//
// The DMA ring is never drained between tiles: the next tile's first steps
// are in flight while the current one finishes, and a tile's stores overlap
// the next tile's multiplies.  A wave stores its block and clears its
// accumulators right after the compute phase of a tile's last step; both
// groups do this at the same point of their own phase sequence, so every wave
// still executes the same barriers.
//
// Operands are K-blocked (kblk_off): a step's 256 rows of one operand are one
// contiguous 16 KB run, and each DMA instruction reads one contiguous
// kilobyte (16 rows x 64 bytes).  With row-major operands the same step reads
// 256 half cache lines 2N bytes apart, which measured 12 % slower overall.
template <int NSP>
__global__ __launch_bounds__(512) void k2_contract_ppp(const bf16* __restrict__ A,
                                                       const bf16* __restrict__ Bm,
                                                       bf16* __restrict__ O, int N, int total)
{
    using namespace k2big;
    constexpr int NW = 8;
    constexpr int DPO = OPB / 1024 / NW;            // DMA instructions per wave per operand (2)
    constexpr int DPS = 2 * DPO;                    // per wave per step
    constexpr int DIST = NSP - 1;                   // DMA runs this many steps ahead
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NSP * STB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;        // group = wm
    const size_t slab = (size_t)N * N;
    const int tiles = (N + BM - 1) / BM;
    const int per_bc = tiles * tiles;
    const int G = gridDim.x, g = blockIdx.x;
    const int n_my = (total - g + G - 1) / G;       // tiles of this workgroup (g < total)
    const int nk = (N + BK - 1) / BK;
    const int S = n_my * nk;                        // steps of this workgroup (< 2^31)

    // Tile tl of this workgroup: virtual block g + tl*G through the XCD-banded
    // order, a bijection of [0, total) because total is a multiple of 8 (C is);
    // with G a multiple of 8 every tile of workgroup g lies in g's band.
    auto tile_geo = [&](int tl, size_t& bc, int& i0, int& j0) {
        const unsigned vb = (unsigned)g + (unsigned)tl * (unsigned)G;
        const unsigned logical = (vb & 7u) * ((unsigned)total >> 3) + (vb >> 3);
        bc = logical / per_bc;
        const int t = (int)(logical % per_bc);
        constexpr int GM = 8;
        const int first_i = (t / (GM * tiles)) * GM;
        const int gm = min(GM, tiles - first_i);
        i0 = (first_i + (t % (GM * tiles)) % gm) * BM;
        j0 = ((t % (GM * tiles)) / gm) * BN;
    };

    // Operand slab: [nk][N][32] bf16.  DMA instruction q of a wave covers rows
    // 16 (DPO wave + q) .. +15 of the tile, one contiguous kilobyte of the
    // step's block; lane l reads row dr, chunk dc (the slot swizzle is
    // applied by choosing which lane reads which chunk).
    const size_t aslab = ab_slab_elems(DType::BF16, N);
    const unsigned nrec = (unsigned)(aslab * sizeof(bf16));
    const int dpos = (lane & 7) ^ (lane >> 3);
    const int dr = 2 * (lane >> 3) + (dpos >> 2), dc = dpos & 3;
    constexpr unsigned qstride = 16u * ROWB;
    const unsigned kstride = (unsigned)N * ROWB;    // bytes per K-block
    const unsigned lane_off = (unsigned)(wave * 16 * DPO + dr) * ROWB + dc * 16u;
    // B rows are loaded permuted within each 32-row group: slot row 16 h + r
    // (h = 0, 1; r = 0..15) holds tile row 8 (r / 4) + 4 h + r % 4.  After the
    // MFMAs of blocks 2p and 2p + 1, lane group g then holds the results for
    // rows 32 p + 8 g .. + 7 of its wave's 64, eight consecutive j of one i,
    // stored as one 16-byte run.  Instruction q of a wave fills slot rows
    // 16 (2 wave + q) .. + 15, i.e. h = q and group wave.
    static_assert(DPO == 2, "B row permutation assumes two DMA instructions per operand per wave");
    const unsigned lane_off_b = (unsigned)(32 * wave + 8 * (dr >> 2) + (dr & 3)) * ROWB + dc * 16u;

    // DMA cursor: the next step to load is K-step ikk of tile itl.  The tile's
    // buffer descriptors and row offsets are recomputed only when the cursor
    // enters a new tile; past the workgroup's last tile (and for K-chunks past
    // N) the offset is pushed beyond the buffer's range, so the DMA reads zeros.
    int itl = 0, ikk = 0;
    __amdgpu_buffer_rsrc_t ra, rb;
    unsigned oa_t = 0, ob_t = 0;
    bool ilive = true;
    auto set_tile = [&]() {
        ilive = itl < n_my;
        size_t bc; int i0, j0;
        tile_geo(ilive ? itl : 0, bc, i0, j0);
        ra = __builtin_amdgcn_make_buffer_rsrc((void*)(A + bc * aslab), 0, nrec, 0x00020000);
        rb = __builtin_amdgcn_make_buffer_rsrc((void*)(Bm + bc * aslab), 0, nrec, 0x00020000);
        oa_t = lane_off + (unsigned)i0 * ROWB;
        ob_t = lane_off_b + (unsigned)j0 * ROWB;
    };
    set_tile();
    int isl = 0;                                    // ring slot of the next step
    auto issue = [&]() {
        unsigned char* st = smem + isl * STB + wave * DPO * 1024;
        const int k0 = ikk * BK;
        const unsigned kb = (unsigned)ikk * kstride;
        const unsigned kpen = (ilive && k0 + dc * 8 < N) ? 0u : 0x80000000u;
#pragma unroll
        for (int q = 0; q < DPO; ++q) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, TRIMUL_LDS_PTR(st + q * 1024), 16,
                                                     (oa_t + q * qstride + kb) | kpen, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, TRIMUL_LDS_PTR(st + OPB + q * 1024), 16,
                                                     (ob_t + q * 4u * ROWB + kb) | kpen, 0, 0, 0);
        }
        if (++isl == NSP) isl = 0;
        if (++ikk == nk) { ikk = 0; ++itl; set_tile(); }
    };

    const int rchunk = lane >> 4;
    const int fa_base = slot_off(wm * 128 + (lane & 15), rchunk);
    const int fb_base = OPB + slot_off(wn * 64 + (lane & 15), rchunk);

    f32x4 acc[8][4];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 fa[8], fb[4];
    auto barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

#pragma unroll
    for (int s0 = 0; s0 < DIST; ++s0) issue();
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((DIST - 1) * DPS));   // own share of step 0 landed
    barrier();                                          // ... everyone's
    if (wm == 1) barrier();                             // group 1 starts one phase late

    int kin = 0;                                        // step within the current tile
    int tl = 0;
    int rsl = 0;                                        // ring slot of step s
    for (int s = 0; s < S; ++s) {
        // M_s
        const unsigned char* st = smem + rsl * STB;
        if (++rsl == NSP) rsl = 0;
#pragma unroll
        for (int m = 0; m < 8; ++m) fa[m] = *reinterpret_cast<const u32x4*>(st + fa_base + m * 1024);
#pragma unroll
        for (int n = 0; n < 4; ++n) fb[n] = *reinterpret_cast<const u32x4*>(st + fb_base + n * 1024);
        issue();                                        // step s + DIST
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lds0((DIST - 1) * DPS));
        barrier();
        // C_s.  Operands swapped (b rows as the MFMA's A): each lane's four
        // results are four consecutive j of one i.
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int n = 0; n < 4; ++n) acc[m][n] = Elem<bf16>::mma(fb[n], fa[m], acc[m][n]);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm((DIST - 1) * DPS));
        barrier();
        if (++kin == nk) {
            // Tile tl complete: store this wave's block and start the next.
            size_t bc; int i0, j0;
            tile_geo(tl, bc, i0, j0);
            bf16* Ob = O + bc * slab;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int i = i0 + wm * 128 + m * 16 + (lane & 15);
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    // j .. j + 7 (8 divides N, so all or none exist)
                    const int j = j0 + wn * 64 + 32 * p + 8 * (lane >> 4);
                    bf16x8 h;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        h[e] = (bf16)acc[m][2 * p][e];
                        h[4 + e] = (bf16)acc[m][2 * p + 1][e];
                    }
                    if (i < N && j < N) *reinterpret_cast<bf16x8*>(Ob + (size_t)i * N + j) = h;
                    acc[m][2 * p] = f32x4{0.f, 0.f, 0.f, 0.f};
                    acc[m][2 * p + 1] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
            kin = 0;
            ++tl;
        }
    }
    if (wm == 0) barrier();                             // balance group 1's extra barrier
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));          // no DMA may outlive the workgroup
}

template <typename T, int BM, int BN>
static hipError_t launch_k2(const void* a, const void* b, int B, int C, int N, void* o,
                            hipStream_t s)
{
    const int tiles_i = (N + BM - 1) / BM, tiles_j = (N + BN - 1) / BN;
    dim3 grid((unsigned)((size_t)tiles_i * tiles_j * B * C));
    hipLaunchKernelGGL((k2_contract<T, BM, BN>), grid, dim3(256), 0, s,
                       (const T*)a, (const T*)b, (T*)o, N, tiles_j);
    return hipGetLastError();
}

hipError_t launch_contract(const Params& p, const void* a_cm, const void* b_cm, int B, int N,
                           void* o, hipStream_t s)
{
    // bf16: the persistent 256 x 256 kernel at every N (measured faster than
    // 128 x 128 tiles down to N = 384 as well: 0.031 against 0.036 ms for
    // C = 128, N = 384); ragged tiles read zeros or rows whose outputs are
    // never stored.
    if (p.dtype == DType::BF16) {
        const int tiles = (N + k2big::BM - 1) / k2big::BM;
        const long long total = (long long)tiles * tiles * B * p.C;
        int dev = 0, cus = 256;
        if (hipGetDevice(&dev) == hipSuccess)
            (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        const long long pg = total < cus ? total : cus;
        hipLaunchKernelGGL(k2_contract_ppp<4>, dim3((unsigned)pg), dim3(512), 0, s, (const bf16*)a_cm,
                           (const bf16*)b_cm, (bf16*)o, N, (int)total);
        return hipGetLastError();
    }
    return launch_k2<float, 128, 128>(a_cm, b_cm, B, p.C, N, o, s);
}

}  // namespace trimul
