// trimul_plans.hpp -- per-shape kernel plans: the candidates trimul_tune
// measures, and the on-disk cache that keeps the winners across processes.
//
// The fold-cp-ops README's single-device path is autotuned and keeps its
// tuning results in an on-disk store separate from its compile cache
// ("Environment": the same code measured cold against warm differs by about
// 2x on an autotuning path).  Here the kernels are compiled ahead of time, so
// only the tuning result is cached: for one device kind, one layer width
// (D, C, dtype) and one call shape (B, N, direction, masked), which Plan ran
// fastest.  Host code only.
#pragma once

#include <string>
#include <vector>

#include "trimul_launch.hpp"

namespace trimul {

struct PlanKey {
    int B, N, dir, masked;
    bool operator==(const PlanKey& o) const
    {
        return B == o.B && N == o.N && dir == o.dir && masked == o.masked;
    }
};

struct PlanEntry {
    PlanKey key;
    Plan plan;
    double ms;   // measured time of the projection and contraction with this plan
};

// The projection variants and the contraction choices trimul_tune times
// (each kernel is timed on its own, and the fastest of each kept).
std::vector<int> k1_variants();
std::vector<Plan> k2_choices();
// Every combination, the default for 256-row tiles first.
std::vector<Plan> candidate_plans();

// The plan of a call shape nothing was recorded for: 256-row tiles in groups
// of 8 row panels, per-round XCD blocks (order 1), which keep all XCDs on the
// same channels (with the two-step contraction, K2 ms on one box, order 1
// against XCD bands: 24.60 against 24.90 at N = 4096, D = C = 256; 98.6
// against 99.9 at N = 8192, D = C = 128; 0.52 against 0.56 at B = 2, N =
// 1024; 3.55 against 3.49 at N = 2048; masked N = 8192 with the live-first
// tile lists: 93.7 against 96.5).  At N <= 512 that is not a multiple of 256,
// 128-row tiles in XCD bands: 256-row tiles would be mostly padding (N = 384:
// 0.028 against 0.032 ms unmasked, 0.0335 against 0.0345 ms masked); where N
// fills 256-row tiles, they are faster (N = 512, D = C = 256: 0.091 against
// 0.121 ms).
Plan default_plan(const PlanKey& k);

// Whether a plan is one of the candidates (plans read from a file or set by a
// test are checked against this before use).
bool plan_valid(const Plan& p);

// Cache file: $TRIMUL_PLAN_CACHE if set ("" or "0" disables the cache), else
// $XDG_CACHE_HOME/libtrimul/plans.txt, else $HOME/.cache/libtrimul/plans.txt;
// "" when disabled or no location is known.
std::string plan_cache_path();

// Device key of the cache: the architecture name without feature suffixes
// and the compute-unit count, e.g. "gfx950-256cu".
std::string plan_device_key(const char* gcn_arch_name, int cus);

// Append to `out` every valid entry of the file recorded for (device, D, C,
// dtype).  Malformed lines are skipped.  Returns false if the file cannot be
// read (a missing file is not an error: returns true with nothing added).
bool plan_cache_load(const std::string& path, const std::string& device, int D, int C, int dtype,
                     std::vector<PlanEntry>& out);

// Record one entry, replacing any line with the same (device, D, C, dtype,
// key).  Writes a temporary file next to `path` and renames it over `path`,
// creating the directory if needed.  Returns false on any I/O failure.
bool plan_cache_store(const std::string& path, const std::string& device, int D, int C, int dtype,
                      const PlanEntry& e);

}  // namespace trimul
