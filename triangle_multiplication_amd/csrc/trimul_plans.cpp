// trimul_plans.cpp -- candidate plans and the on-disk plan cache (host only).
//
// File format: plain text, one entry per line, fields separated by spaces:
//   trimul-plan v3 <device> <D> <C> <dtype> <B> <N> <dir> <masked> <k1_variant> <k2_order> <k2_gm> <k2_tile> <ms>
// dtype 0 = bf16, 1 = fp32; dir 0 = outgoing, 1 = incoming; masked 0 or 1.
// Lines starting with '#' and lines that do not parse are ignored.
#include "trimul_plans.hpp"

#include <sys/stat.h>
#include <unistd.h>

#include <cerrno>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <sstream>

namespace trimul {

std::vector<int> k1_variants() { return {0}; }

std::vector<Plan> k2_choices()
{
    std::vector<Plan> v;
    for (int tile : {256, 128})
        for (int order : {1, 0})
            for (int gm : {8, 4, 16}) {
                Plan p;
                p.k2_order = order;
                p.k2_gm = gm;
                p.k2_tile = tile;
                v.push_back(p);
            }
    return v;
}

std::vector<Plan> candidate_plans()
{
    std::vector<Plan> v;
    for (int k1 : k1_variants())
        for (Plan p : k2_choices()) {
            p.k1_variant = k1;
            v.push_back(p);
        }
    return v;
}

Plan default_plan(const PlanKey& k)
{
    Plan p;
    if (k.N <= 512 && k.N % 256 != 0)
        p.k2_tile = 128;          // 128-row tiles walk the plain order, masked or not
    else
        p.k2_order = 1;
    return p;
}

bool plan_valid(const Plan& p)
{
    for (const Plan& c : candidate_plans())
        if (c.k1_variant == p.k1_variant && c.k2_order == p.k2_order && c.k2_gm == p.k2_gm &&
            c.k2_tile == p.k2_tile)
            return true;
    return false;
}

std::string plan_cache_path()
{
    const char* env = std::getenv("TRIMUL_PLAN_CACHE");
    if (env) {
        if (!*env || std::strcmp(env, "0") == 0) return "";
        return env;
    }
    const char* xdg = std::getenv("XDG_CACHE_HOME");
    if (xdg && *xdg) return std::string(xdg) + "/libtrimul/plans.txt";
    const char* home = std::getenv("HOME");
    if (home && *home) return std::string(home) + "/.cache/libtrimul/plans.txt";
    return "";
}

std::string plan_device_key(const char* gcn_arch_name, int cus)
{
    std::string a = gcn_arch_name ? gcn_arch_name : "unknown";
    const size_t colon = a.find(':');
    if (colon != std::string::npos) a.resize(colon);
    return a + "-" + std::to_string(cus) + "cu";
}

namespace {

struct Line {
    std::string device;
    int D, C, dtype;
    PlanEntry e;
};

bool parse_line(const std::string& text, Line& L)
{
    std::istringstream in(text);
    std::string tag, ver;
    if (!(in >> tag >> ver) || tag != "trimul-plan" || ver != "v3") return false;
    if (!(in >> L.device >> L.D >> L.C >> L.dtype >> L.e.key.B >> L.e.key.N >> L.e.key.dir >>
          L.e.key.masked >> L.e.plan.k1_variant >> L.e.plan.k2_order >> L.e.plan.k2_gm >> L.e.plan.k2_tile >>
          L.e.ms))
        return false;
    return plan_valid(L.e.plan) && L.e.key.B >= 1 && L.e.key.N >= 1 && (L.e.key.dir == 0 || L.e.key.dir == 1) &&
           (L.e.key.masked == 0 || L.e.key.masked == 1);
}

std::string format_line(const std::string& device, int D, int C, int dtype, const PlanEntry& e)
{
    char buf[256];
    std::snprintf(buf, sizeof buf, "trimul-plan v3 %s %d %d %d %d %d %d %d %d %d %d %d %.6g", device.c_str(), D,
                  C, dtype, e.key.B, e.key.N, e.key.dir, e.key.masked, e.plan.k1_variant, e.plan.k2_order,
                  e.plan.k2_gm, e.plan.k2_tile, e.ms);
    return buf;
}

bool mkdir_p(const std::string& dir)
{
    if (dir.empty()) return true;
    struct stat st;
    if (stat(dir.c_str(), &st) == 0) return S_ISDIR(st.st_mode);
    const size_t slash = dir.find_last_of('/');
    if (slash != std::string::npos && slash > 0 && !mkdir_p(dir.substr(0, slash))) return false;
    return mkdir(dir.c_str(), 0755) == 0 || errno == EEXIST;
}

}  // namespace

bool plan_cache_load(const std::string& path, const std::string& device, int D, int C, int dtype,
                     std::vector<PlanEntry>& out)
{
    if (path.empty()) return true;
    std::ifstream f(path);
    if (!f) return errno == ENOENT;
    std::string text;
    while (std::getline(f, text)) {
        Line L;
        if (!parse_line(text, L) || L.device != device || L.D != D || L.C != C || L.dtype != dtype) continue;
        bool replaced = false;
        for (PlanEntry& e : out)
            if (e.key == L.e.key) {
                e = L.e;   // later lines win
                replaced = true;
            }
        if (!replaced) out.push_back(L.e);
    }
    return true;
}

bool plan_cache_store(const std::string& path, const std::string& device, int D, int C, int dtype,
                      const PlanEntry& e)
{
    if (path.empty()) return false;
    const size_t slash = path.find_last_of('/');
    if (slash != std::string::npos && !mkdir_p(path.substr(0, slash))) return false;
    std::vector<std::string> keep;
    {
        std::ifstream f(path);
        std::string text;
        while (f && std::getline(f, text)) {
            Line L;
            if (parse_line(text, L) && L.device == device && L.D == D && L.C == C && L.dtype == dtype &&
                L.e.key == e.key)
                continue;   // replaced below
            keep.push_back(text);
        }
    }
    keep.push_back(format_line(device, D, C, dtype, e));
    const std::string tmp = path + ".tmp" + std::to_string((long)getpid());
    {
        std::ofstream o(tmp, std::ios::trunc);
        if (!o) return false;
        for (const std::string& l : keep) o << l << '\n';
        o.flush();
        if (!o) {
            std::remove(tmp.c_str());
            return false;
        }
    }
    if (std::rename(tmp.c_str(), path.c_str()) != 0) {
        std::remove(tmp.c_str());
        return false;
    }
    return true;
}

}  // namespace trimul
