// Record of the launches the host code asked for (host-only checks).
#pragma once
#include <string>
#include <vector>

struct Launch {
    std::string kind;
    int p0, p1, wpos, window, n_cls;
};

struct LaunchLog {
    std::vector<Launch> v;
    void add(const char *k, int p0, int p1, int wpos, int window, int n_cls) {
        v.push_back({k, p0, p1, wpos, window, n_cls});
    }
    void clear() { v.clear(); }
};

extern LaunchLog g_launches;
