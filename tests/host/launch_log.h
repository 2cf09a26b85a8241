// Record of the launches the host code asked for (host-only checks).
#pragma once
#include <string>
#include <vector>

#include <hip/hip_runtime_api.h>

struct Launch {
    std::string kind;
    int p0, p1, wpos, window, n_cls;
    int n_rb, Hc[2], groups[2];        // task bookkeeping of a step launch
    int win_pc;                        // windowed launches: per-channel decays
};

struct LaunchLog {
    std::vector<Launch> v;
    void add(const char *k, int p0, int p1, int wpos, int window, int n_cls, int n_rb = 0,
             const int *Hc = nullptr, const int *groups = nullptr, int win_pc = 0) {
        Launch l{k, p0, p1, wpos, window, n_cls, n_rb, {0, 0}, {0, 0}, win_pc};
        for (int i = 0; i < 2 && Hc; ++i) {
            l.Hc[i] = Hc[i];
            l.groups[i] = groups[i];
        }
        v.push_back(l);
    }
    void clear() { v.clear(); }
};

extern LaunchLog g_launches;

// The stand-in sticky HIP error (launch_stubs.cpp): an error left by earlier
// work on the thread, and a switch that makes the next stand-in launch fail.
extern hipError_t g_sticky_error;
extern bool g_fail_next_launch;
