"""Decode-time attention of a few queries against a large cached K/V, on MI355X.

Importing this package loads nothing native; the HIP library is opened on the
first call into it (see ``ops``)."""
